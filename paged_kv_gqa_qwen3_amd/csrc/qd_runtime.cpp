// Host runtime of libqd: handle, weight repack, step orchestration and one
// captured hipGraph per (batch size, pointer set).
//
// The graph design follows the pages' decode-graph pattern ("GPU 算子与执行优化",
// Part 5: dynamic metadata stays outside, addresses inside the graph are
// frozen; "突破vLLM推理性能瓶颈", section 2: one graph per batch size) with one
// change: the split-KV partition count is derived on the device from the
// positions, so a single graph per batch size serves every context length
// (the blog's Part 8 had to leave graphs above 2048 tokens because a frozen
// grid fixed the split count).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "qd.h"
#include "qd_internal.h"
#include "qd_stream_plan.h"

using namespace qd;

namespace {

std::string g_create_error;

struct GraphKey {
  int B;
  const void* p[6];
  bool operator<(const GraphKey& o) const {
    if (B != o.B) return B < o.B;
    return std::memcmp(p, o.p, sizeof(p)) < 0;
  }
};

// Captured graphs a handle keeps (one per batch size and pointer set).
constexpr int kMaxGraphs = 64;

struct GemvPlan {
  int S = 1, kps = 1, rt = 4;
  bool wide = false;  // chunk-streamed items (gemv_wide_item), rt = 8
};

struct LayerW {
  uint16_t *qkv = nullptr, *o = nullptr, *gu = nullptr, *down = nullptr;
  float *in_norm = nullptr, *post_norm = nullptr, *q_norm = nullptr, *k_norm = nullptr;
};

}  // namespace

struct qd_handle {
  qd_config cfg{};
  hipStream_t stream = nullptr;
  hipStream_t cap = nullptr;
  int device = 0;
  int num_cus = 256;
  std::string err;

  int L = 0, H = 0, Hq = 0, Hkv = 0, D = 0, I = 0, V = 0, QD = 0, KD = 0, NQKV = 0, G = 0;
  std::vector<void*> allocs;
  std::vector<LayerW> lw;
  uint16_t* embed = nullptr;
  uint16_t* lm = nullptr;
  float* final_norm = nullptr;
  std::map<std::string, int> expected;  // name -> loaded (0/1)

  float *x = nullptr, *ssq = nullptr, *qkv = nullptr, *attn = nullptr, *act = nullptr;
  // bf16 pairs [64][cols] for MFMA consumers (batch >= 2)
  uint16_t *xg_hi = nullptr, *xg_lo = nullptr, *attn_hi = nullptr, *attn_lo = nullptr;
  uint16_t *act_hi = nullptr, *act_lo = nullptr;
  // the fused MLP launch: the second residual / norm / MFMA-pair set (down
  // writes the next layer's while gate/up items of the same launch still
  // read this layer's), down's own split partials and counters, and two
  // alternating sets of completion counters, kCntStride apart
  float *x_b = nullptr, *ssq_b = nullptr;
  uint16_t *xg_b_hi = nullptr, *xg_b_lo = nullptr;
  float* part_b = nullptr;
  unsigned* gemv_cnt_b = nullptr;
  unsigned* fused_cnt = nullptr;
  int fused_cnt_n = 0;
  float* part = nullptr;      // split partials of self-reducing projections (O, down, LM head)
  float* part_qkv = nullptr;  // split partials of QKV, summed by attention
  unsigned* gemv_cnt = nullptr;
  float *o_part = nullptr, *ml_part = nullptr;
  unsigned* attn_cnt = nullptr;
  float* amax_val = nullptr;
  int* amax_idx = nullptr;
  float* amax_val2 = nullptr;
  int* amax_idx2 = nullptr;
  unsigned* amax_cnt = nullptr;
  int32_t* prof_ids = nullptr;  // next-token output of qd_profile_class's LM head launches
  // qd_sample scratch: chunk maxima, chunk candidates, per-row arrival counters
  int sample_G = 1, sample_C = 0;
  float* sample_max = nullptr;
  int* sample_idx = nullptr;
  unsigned long long* sample_cand = nullptr;
  unsigned* sample_cnt = nullptr;
  double* sample_sum = nullptr;
  unsigned* sample_cnt2 = nullptr;
  double* sample_hist = nullptr;
  double* sample_pass_hist = nullptr;  // the third sampling launch's buffers
  double *sample_sum2 = nullptr, *sample_sum3 = nullptr;
  unsigned* sample_cnt3 = nullptr;
  int *sample_flag = nullptr, *sample_cut = nullptr;
  int* dev_flags = nullptr;
  float *rope_cos = nullptr, *rope_sin = nullptr;
  int max_pos = 0;

  std::map<GraphKey, hipGraphExec_t> graphs;
  std::map<GraphKey, hipGraph_t> graph_defs;
  std::map<GraphKey, unsigned long long> graph_use;  // last replay, for eviction at the cap
  unsigned long long graph_clock = 0;

  // batch-1 streaming step (persistent handles)
  bool persistent = false;
  bool long_ctx = false;  // max_pages_per_seq > kStreamMaxPages: batch 1 takes the per-stage kernels
  bool mid_ctx = false;   // max_pages_per_seq >= kMidCtxPages: 3 attention pages per wave up to batch 8
  LayerDev* layers_dev = nullptr;
  unsigned* step_cnt = nullptr;
  unsigned* step_flags = nullptr;  // [2 * CUs][32]
  unsigned* step_exit = nullptr;
  unsigned* step_abort = nullptr;
  // batch-1 streaming step (persistent handles whose shapes fit it)
  bool stream_ok = false;
  int stream_grid = 0;
  size_t stream_lds = 0;
  int stream_in_floats = 0, stream_rt_max = 0, stream_res_off = 0, stream_qkv_S = 1;
  StreamRun* stream_runs = nullptr;  // every wave's weight-tile runs
  int* stream_run_off = nullptr;     // [stream_grid][4]
  float* stream_amax_val = nullptr;  // [stream_grid]
  int* stream_amax_idx = nullptr;

  // KV pool elements: bf16, or E4M3 codes with per-tensor scales
  bool kv_fp8 = false;
  int kv_bytes = 2;
  float k_scale = 1.f, v_scale = 1.f;

  // prompt chunks on the matrix cores (qd_prefill_prompts): pf_rows rows of
  // residual stream, QKV output, q pairs and operand tiles (norm outputs and
  // the attention output share pf_tin; the SwiGLU output is pf_tact)
  int pf_rows = 0;
  float* pf_x = nullptr;
  float* pf_qkv = nullptr;
  uint16_t *pf_q_hi = nullptr, *pf_q_lo = nullptr;
  uint16_t* pf_tin = nullptr;
  uint16_t* pf_tact = nullptr;
};

namespace {

int fail(qd_handle* h, int code, const std::string& msg) {
  if (h) h->err = msg; else g_create_error = msg;
  return code;
}

int hip_fail(qd_handle* h, hipError_t e, const char* what) {
  return fail(h, QD_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define HIP_TRY(h, expr)                                  \
  do {                                                    \
    hipError_t e_ = (expr);                               \
    if (e_ != hipSuccess) return hip_fail((h), e_, #expr); \
  } while (0)

template <typename T>
int dev_alloc(qd_handle* h, T** p, size_t count) {
  void* q = nullptr;
  size_t bytes = count * sizeof(T);
  if (bytes == 0) bytes = 16;
  hipError_t e = hipMalloc(&q, bytes);
  if (e != hipSuccess) return fail(h, QD_ENOMEM, std::string("hipMalloc failed: ") + hipGetErrorString(e));
  h->allocs.push_back(q);
  *p = static_cast<T*>(q);
  return QD_OK;
}

// Split plan for an N x K projection at batch B.
//
// Batch 1 (VALU items): one 16-row tile per workgroup, its 4 waves splitting
// K, and K itself split only where the input slice would not fit an 80 KB
// LDS budget or the row tiles alone give fewer than 128 workgroups: the
// projections of a 4B-class model then need no split-K hand-off at batch 1.
// The LM head keeps 64-row items (its argmax reduces one partial per row
// group).
// Batch >= 2 (MFMA items): 64-row items, the fewest K splits that give every
// CU an item, slices of at most 16 k-tiles while the row groups alone do
// not, and an LDS input slice <= 48 KB so that three workgroups fit a CU.
constexpr size_t kLdsCapValu = 80 * 1024;
constexpr size_t kLdsCapStaged = 48 * 1024;
// Wider batches stage more input columns per k-tile: a 48 KB cap would cut K
// into slices of 3 k-tiles at 64 columns, and the split partials (S x N x 64
// floats, written and read back) would outweigh the weights.  A 76 KB cap
// keeps two workgroups per CU and slices of 7-16 k-tiles (4B shape,
// 512-token prompt in 64-row chunks: 249 -> 126 ms, 32-row: 131 -> 100 ms;
// one workgroup per CU with 124 KB: 137 and 112 ms; 16 columns stay best at
// 48 KB).
constexpr size_t gemv_lds_cap(int nb) { return nb >= 32 ? (size_t)76 * 1024 : kLdsCapStaged; }
constexpr int kMinValuItems = 128;

// A persistent handle runs batch 1 as the weight-streaming step kernel when
// its shapes fit and it is sized for short contexts (decided in qd_create);
// every other step takes the per-stage kernels.
bool use_stream(const qd_handle* h, int B) { return h->stream_ok && B == 1; }

// Chunk-streamed items of 128 rows (gemv_wide_item; N a multiple of 128).
GemvPlan plan_wide(const qd_handle* h, int N, int K) {
  GemvPlan p;
  const int KT = K / kTileCols;
  p.rt = 8;
  p.wide = true;
  const int nrg = N / (2 * kRowsPerGroup);
  const int S0 = std::min(KT, std::max(1, (h->num_cus / 2 + nrg - 1) / nrg));
  p.kps = (KT + S0 - 1) / S0;
  p.S = (KT + p.kps - 1) / p.kps;
  return p;
}

GemvPlan plan_gemv(const qd_handle* h, int N, int K, int B, bool argmax = false,
                   bool wide = true) {
  const int KT = K / kTileCols, NRG = N / kRowsPerGroup;
  const int nb = gemv_nb(B);
  GemvPlan p;
  if (nb == 1) {
    // batch 1 (VALU): one 16-row tile per item (the LM head: four), K split
    // only when needed (LDS budget, or fewer than 128 items)
    p.rt = argmax ? 4 : 1;
    const int groups = N / (kTileRows * p.rt);
    for (int S = 1; S <= KT; ++S) {
      const int kps = (KT + S - 1) / S;
      const int Se = (KT + kps - 1) / kps;
      if (gemv_lds_bytes(B, kps, p.rt) > kLdsCapValu && kps > 1) continue;
      p.S = Se;
      p.kps = kps;
      if (groups * Se >= kMinValuItems) return p;
    }
    return p;
  }
  // 32 and 64 columns: chunk-streamed items of 128 rows (rt = 8; two row
  // tiles per wave), K split only until there are items for half the CUs
  // (4B shape, per step at batch 32 / 64: one item per CU 4.22 / 6.14 ms,
  // half 3.73 / 5.44, a third 4.05 / 5.98, one and a half 3.80 / 5.67; one
  // per CU for O and down alone 3.92 / 5.72; four row tiles per wave spill
  // registers: 7.91 / 14.1)
  // The LM head takes them from 8 batch columns up (batch 16: 3.295 ->
  // 3.247 ms per step; batch 8: 2.832 -> 2.819); QKV and O at 8 and 16
  // columns were slower with them (batch 8: 2.85 and 2.85 against 2.83).
  if ((nb >= 32 || argmax) && N % (2 * kRowsPerGroup) == 0) return plan_wide(h, N, K);
  // MFMA items (batch >= 2): the fewest K splits that give every CU an item,
  // slices of at most 16 k-tiles while row groups alone do not (measured on
  // the 4B shape: batch 8 3.39 -> 3.19 ms per step against two items per CU
  // and 20-tile slices; batch 16 4.00 -> 3.93)
  const int mtarget = h->num_cus;
  auto search = [&](int rt, int nrg, GemvPlan& q) {
    q.rt = rt;
    for (int S = 1; S <= KT; ++S) {
      const int kps = (KT + S - 1) / S;
      const int Se = (KT + kps - 1) / kps;
      if (kps > 16 && nrg < mtarget) continue;
      if (gemv_lds_bytes(B, kps, rt) > gemv_lds_cap(nb)) continue;
      q.S = Se;
      q.kps = kps;
      if (nrg * Se >= mtarget) return true;
    }
    if (q.S == 1 && q.kps == 1 && KT > 1) { q.S = KT; q.kps = 1; }
    return false;
  };
  search(4, NRG, p);
  // 16 batch columns: an item's input slice is half the size of its
  // weights, so items of 128 rows (two row tiles per wave, each input
  // operand read once for both) where they still give every CU two items,
  // with at most one more K split.  On the 4B shape that is gate/up alone
  // (760 items instead of 1216: batch 16 3.62 -> 3.51 ms per step); with
  // one item per CU (down, QKV) the CUs keep too few tiles in flight (3.68).
  GemvPlan p8;
  if (nb == 16 && wide && N % (2 * kRowsPerGroup) == 0 &&
      search(8, N / (2 * kRowsPerGroup), p8) && p8.S <= p.S + 1 &&
      (long long)(N / (2 * kRowsPerGroup)) * p8.S >= 2LL * mtarget)
    return p8;
  return p;
}

// Most splits of one sequence (its longest table) at batch B in the
// per-stage attention kernel, and in the streaming kernel's items.
int attn_pw(const qd_handle* h, int B) {
  return attn_pages_per_wave_kv(B, h->long_ctx, h->kv_fp8, h->mid_ctx);
}
int attn_splits(const qd_handle* h, int B) {
  const int pps = kAttnWaves * attn_pw(h, B);
  return std::max(1, (h->cfg.max_pages_per_seq + pps - 1) / pps);
}
int stream_attn_splits(const qd_handle* h) {
  const int pps = attn_pages_per_split(1, true);
  return std::max(1, (h->cfg.max_pages_per_seq + pps - 1) / pps);
}

// Workgroups of the standalone attention kernel: they take the step's items
// round robin; at most two per CU.
int attn_grid(const qd_handle* h, int B) {
  return std::max(1, std::min(2 * h->num_cus, B * h->Hkv * attn_splits(h, B)));
}

// Weight bytes a launch prefetches into the L2s for the next one: three
// quarters of the eight XCDs' 4 MB L2s.  (Batch 8 and 16, with gate/up and
// QKV both prefetched: 24 MB each 2.822 and 3.326 ms per step, 32 MB each
// 2.825 and 3.363, 16 MB of QKV 2.824 and 3.354.)
constexpr long long kL2PrefetchBytes = 24ll << 20;
// Prefetching workgroups: in an attention launch (8 waves each), in a GEMV launch.
constexpr int kPrefetchWgAttn = 128, kPrefetchWgGemv = 256;

// The first items of the GEMV launch that follows (w: N x K, planned p),
// up to kL2PrefetchBytes, for n_wg prefetching workgroups of this launch.
L2Prefetch next_weights(const uint16_t* w, int N, int K, const GemvPlan& p, int n_wg) {
  L2Prefetch f{};
  f.w = w;
  f.KT = K / kTileCols;
  f.rt = p.rt; f.S = p.S; f.kps = p.kps;
  const long long item = (long long)p.rt * p.kps * kTileElems * 2;
  f.items = (int)std::min<long long>((long long)(N / (kTileRows * p.rt)) * p.S,
                                     std::max(1ll, kL2PrefetchBytes / item));
  f.n_wg = n_wg;
  return f;
}

int validate_config(const qd_config* c) {
  if (!c) return fail(nullptr, QD_EINVAL, "config is NULL");
  if (c->num_layers < 1 || c->hidden < 64 || c->num_q_heads < 1 || c->num_kv_heads < 1 ||
      c->head_dim < 1 || c->intermediate < 32 || c->vocab < 64)
    return fail(nullptr, QD_EINVAL, "model sizes must be positive");
  if (c->max_batch < 1 || c->max_batch > kMaxBatch)
    return fail(nullptr, QD_EINVAL, "max_batch must be in 1..64");
  if (c->max_pages_per_seq < 1 || c->num_pages < 1)
    return fail(nullptr, QD_EINVAL, "max_pages_per_seq and num_pages must be >= 1");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.0))
    return fail(nullptr, QD_EINVAL, "rms_eps and rope_theta must be > 0");
  if (c->page_size != kPage) return fail(nullptr, QD_EUNSUPPORTED, "page_size must be 16");
  if (c->max_prefill_rows < 0 || c->max_prefill_rows > kPfMaxRows)
    return fail(nullptr, QD_EINVAL, "max_prefill_rows must be in 0..16384");
  if (c->kv_dtype != 0 && c->kv_dtype != 1)
    return fail(nullptr, QD_EINVAL, "kv_dtype must be 0 (bf16) or 1 (E4M3)");
  if (c->kv_dtype == 1 && !(c->k_scale > 0.f && c->v_scale > 0.f && std::isfinite(c->k_scale) &&
                            std::isfinite(c->v_scale)))
    return fail(nullptr, QD_EINVAL, "k_scale and v_scale must be finite and > 0");
  if (c->hidden % 64 || c->hidden > 8192)
    return fail(nullptr, QD_EUNSUPPORTED, "hidden must be a multiple of 64 and at most 8192");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(nullptr, QD_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (c->num_q_heads % c->num_kv_heads)
    return fail(nullptr, QD_EUNSUPPORTED, "num_q_heads must be a multiple of num_kv_heads");
  const int G = c->num_q_heads / c->num_kv_heads;
  if (G != 1 && G != 2 && G != 4)
    return fail(nullptr, QD_EUNSUPPORTED, "query heads per KV head must be 1, 2 or 4");
  if (c->intermediate % 32) return fail(nullptr, QD_EUNSUPPORTED, "intermediate must be a multiple of 32");
  if (c->vocab % 64) return fail(nullptr, QD_EUNSUPPORTED, "vocab must be a multiple of 64");
  // (every split's (max, sum) pair of one sequence is staged in LDS by the combine)
  constexpr int kMaxPages =
      kMaxSplitsStaged * std::min(attn_pages_per_split(1, false), attn_pages_per_split(1, true));
  if ((long long)c->max_pages_per_seq > (long long)kMaxPages)
    return fail(nullptr, QD_EUNSUPPORTED, "max_pages_per_seq too large");
  return QD_OK;
}

struct StepPtrs {
  int B;
  const int32_t* tokens;
  const int32_t* positions;
  const int32_t* tables;
  unsigned char* pool;  // the caller's pool, as bytes
  int32_t* next;
  float* logits;
  int n_logits = -1;  // a prefill chunk: rows [0, n_logits) get the LM head; -1: a decode step
};

// Optional per-launch event recording (qd_profile_step).
struct Prof {
  std::vector<hipEvent_t> ev;  // ev[0] before the first launch, ev[i+1] after launch i
  std::vector<int> cls;        // class of launch i
};

int prof_mark(qd_handle* h, Prof* pr, int cls, hipStream_t s) {
  if (!pr) return QD_OK;
  hipEvent_t e = nullptr;
  HIP_TRY(h, hipEventCreate(&e));
  pr->ev.push_back(e);
  pr->cls.push_back(cls);
  HIP_TRY(h, hipEventRecord(e, s));
  return QD_OK;
}

#ifdef QD_STEP_TRACE
// (trace builds) per-item event timestamps of layer kTraceLayer's launches of
// an eager step, by class (QD_PROF_*), written to QD_TRACE_OUT after it
constexpr int kTraceLayer = 17;
constexpr size_t kTraceSlots = (size_t)kTraceItems * 8;
unsigned long long* g_trace[QD_PROF_CLASSES];
#endif

// The pool's element type and scales, for an attention launch.
void set_kv(const qd_handle* h, AttnArgs& a) {
  a.kv_fp8 = h->kv_fp8 ? 1 : 0;
  a.k_scale = h->k_scale; a.v_scale = h->v_scale;
  a.k_inv = 1.f / h->k_scale; a.v_inv = 1.f / h->v_scale;
}

// Launch the projection of class cls (QD_PROF_QKV, _O, _GATE_UP, _DOWN or
// _LM_HEAD) of layer l at batch B on stream s, as the step does.  QKV leaves
// split partials for attention when part_mode (else it stores q|k|v).
// MFMA consumers (batch >= 2) read the bf16 pairs their producer wrote once:
// x times the next RMSNorm gain (xg), the attention output, act.
hipError_t launch_projection(qd_handle* h, int B, int cls, int l, bool part_mode, float* logits,
                             int32_t* next, hipStream_t s) {
  const int H = h->H, L = h->L;
  const bool mfma = gemv_mfma(B);
  uint16_t* const xg[2] = {h->xg_hi, h->xg_lo};
  uint16_t* const attn_hl[2] = {h->attn_hi, h->attn_lo};
  uint16_t* const act_hl[2] = {h->act_hi, h->act_lo};
  // xin_hl: the MFMA input pairs; out_hl/out_gain: pairs this projection
  // writes for the next MFMA consumer
  auto gemv = [&](const uint16_t* w, int N, int K, const float* xin, uint16_t* const* xin_hl,
                  const float* gain, int mode, float* out, uint16_t* const* out_hl = nullptr,
                  const float* out_gain = nullptr) -> hipError_t {
    GemvPlan p = plan_gemv(h, N, K, B, mode == kArgmax);
    GemvArgs a{};
    a.w = w; a.N = N; a.K = K; a.B = B; a.Bmax = h->cfg.max_batch;
    a.S = p.S; a.kps = p.kps; a.rt = p.rt; a.wide = p.wide ? 1 : 0;
    a.x = xin;
    if (mfma) {
      a.xh = xin_hl[0]; a.xl = xin_hl[1];
      if (out_hl) { a.xo_hi = out_hl[0]; a.xo_lo = out_hl[1]; a.xo_gain = out_gain; }
    }
    a.ssq = gain ? h->ssq : nullptr;
    a.gain = gain; a.eps = h->cfg.rms_eps;
    a.dev_flags = h->dev_flags;
    a.part = mode == kPartial ? h->part_qkv : h->part;
    a.counters = h->gemv_cnt;
    a.out = out;
    a.ssq_out = h->ssq;
    a.logits = logits;
    a.amax_val = h->amax_val; a.amax_idx = h->amax_idx; a.amax_counter = h->amax_cnt;
    a.amax_val2 = h->amax_val2; a.amax_idx2 = h->amax_idx2;
    a.next_ids = next;
#ifdef QD_STEP_TRACE
    if (l == kTraceLayer || (cls == QD_PROF_LM_HEAD && g_trace[cls] != nullptr))
      a.trace = g_trace[cls];
#endif
    return launch_gemv(a, mode, s);
  };
  if (cls == QD_PROF_LM_HEAD) return gemv(h->lm, h->V, H, h->x, xg, h->final_norm, kArgmax, nullptr);
  const LayerW& w = h->lw[l];
  switch (cls) {
    case QD_PROF_QKV:
      return gemv(w.qkv, h->NQKV, H, h->x, xg, w.in_norm, part_mode ? kPartial : kStore, h->qkv);
    case QD_PROF_O:
      return gemv(w.o, H, h->QD, h->attn, attn_hl, nullptr, kResid, h->x, xg, w.post_norm);
    case QD_PROF_GATE_UP:
      return gemv(w.gu, 2 * h->I, H, h->x, xg, w.post_norm, kSwiGLU, h->act, act_hl);
    case QD_PROF_DOWN:
      return gemv(w.down, H, h->I, h->act, act_hl, nullptr, kResid, h->x, xg,
                  l + 1 < L ? h->lw[l + 1].in_norm : h->final_norm);
    default:
      return hipErrorInvalidValue;
  }
}

// Enqueue one step on stream s.
int record_step_fused(qd_handle* h, const StepPtrs& sp, hipStream_t s);

int record_step(qd_handle* h, const StepPtrs& sp, const qd_taps* taps, hipStream_t s,
                Prof* pr = nullptr) {
  // a decode step at batches 2-16 runs the MLP half of every layer as one
  // fused launch (the taps, profiling and prefill paths keep one launch per
  // stage)
  if (taps == nullptr && pr == nullptr && sp.n_logits < 0 && fused_supported(sp.B))
    return record_step_fused(h, sp, s);
  int prc = QD_OK;
  if (pr && (prc = prof_mark(h, pr, -1, s))) return prc;
#define PROF(c)                                              \
  do {                                                       \
    if (pr && (prc = prof_mark(h, pr, (c), s))) return prc;  \
  } while (0)
  const int B = sp.B, L = h->L, H = h->H;
  const float eps = h->cfg.rms_eps;
  const size_t layer_elems = (size_t)h->cfg.num_pages * 2 * h->Hkv * kPage * h->D;
  const bool mfma = gemv_mfma(B);
#ifdef QD_STEP_TRACE
  hipStreamCaptureStatus cap_st = hipStreamCaptureStatusNone;
  (void)hipStreamIsCapturing(s, &cap_st);
  const bool tracing = std::getenv("QD_TRACE_OUT") != nullptr && cap_st == hipStreamCaptureStatusNone;
  for (int c = 0; c < QD_PROF_CLASSES; ++c) {
    if (tracing && g_trace[c] == nullptr) HIP_TRY(h, hipMalloc(&g_trace[c], kTraceSlots * 8));
    if (tracing) HIP_TRY(h, hipMemsetAsync(g_trace[c], 0xff, kTraceSlots * 8, s));
  }
  if (!tracing)
    for (int c = 0; c < QD_PROF_CLASSES; ++c) g_trace[c] = nullptr;
#endif

  EmbedArgs ea{};
  ea.table = h->embed;
  ea.V = h->V; ea.H = H; ea.B = B; ea.Bmax = h->cfg.max_batch;
  ea.tokens = sp.tokens; ea.x = h->x; ea.ssq_out = h->ssq; ea.dev_flags = h->dev_flags;
  if (mfma) { ea.xo_hi = h->xg_hi; ea.xo_lo = h->xg_lo; ea.xo_gain = h->lw[0].in_norm; }
  HIP_TRY(h, launch_embed(ea, s));
  PROF(QD_PROF_EMBED);

  auto proj = [&](int cls, int l, bool part_mode) {
    return launch_projection(h, B, cls, l, part_mode, sp.logits, sp.next, s);
  };
  const int smax = attn_splits(h, B);
  for (int l = 0; l < L; ++l) {
    const LayerW& w = h->lw[l];
    const bool tap = taps && taps->layer == l;
    if (tap && taps->x_in)
      HIP_TRY(h, hipMemcpyAsync(taps->x_in, h->x, sizeof(float) * B * H, hipMemcpyDeviceToDevice, s));
    // Without taps, QKV leaves split partials that attention sums when it
    // reads q, k, v (same order as the finalising mode, so the bits agree);
    // with taps the projection is materialised for checking.
    const bool part_mode = taps == nullptr;
    const GemvPlan pq = plan_gemv(h, h->NQKV, H, B);
    HIP_TRY(h, proj(QD_PROF_QKV, l, part_mode));
    PROF(QD_PROF_QKV);
    if (tap && taps->qkv)
      HIP_TRY(h, hipMemcpyAsync(taps->qkv, h->qkv, sizeof(float) * B * h->NQKV,
                                hipMemcpyDeviceToDevice, s));
    AttnArgs aa{};
    aa.qkv = h->qkv; aa.q_gain = w.q_norm; aa.k_gain = w.k_norm;
    if (part_mode) { aa.qkv_part = h->part_qkv; aa.qkv_S = pq.S; aa.qkv_rows = kTileRows * pq.rt; }
    aa.rope_cos = h->rope_cos; aa.rope_sin = h->rope_sin; aa.max_pos = h->max_pos;
    aa.pool_layer = sp.pool + (size_t)l * layer_elems * h->kv_bytes;
    set_kv(h, aa);
    aa.num_pages = h->cfg.num_pages;
    aa.positions = sp.positions; aa.block_tables = sp.tables;
    aa.max_pages = h->cfg.max_pages_per_seq;
    aa.B = B; aa.Hq = h->Hq; aa.Hkv = h->Hkv;
    aa.eps = eps; aa.scale = (float)(1.0 / std::sqrt((double)h->D));
    aa.S_max = smax;
    aa.grid = attn_grid(h, B);
    aa.o_part = h->o_part; aa.ml_part = h->ml_part; aa.counters = h->attn_cnt;
    aa.out = h->attn;
    if (mfma) { aa.out_hi = h->attn_hi; aa.out_lo = h->attn_lo; }
    aa.tap_q = tap ? taps->q_rot : nullptr;
    aa.tap_k = tap ? taps->k_rot : nullptr;
    aa.dev_flags = h->dev_flags;
#ifdef QD_STEP_TRACE
    if (l == kTraceLayer) aa.trace = g_trace[QD_PROF_ATTN];
#endif
    if (sp.n_logits >= 0) {  // prefill: every row's k, v in the pool before any row attends
      aa.kv_mode = kAppendOnly;
      HIP_TRY(h, launch_attention(aa, h->D, h->G, kAttnWaves,
                                  attn_pw(h, B), s));
      aa.kv_mode = kAttendOnly;
    }
    HIP_TRY(h, launch_attention(aa, h->D, h->G, kAttnWaves,
                                attn_pw(h, B), s));
    PROF(QD_PROF_ATTN);
    if (tap && taps->attn)
      HIP_TRY(h, hipMemcpyAsync(taps->attn, h->attn, sizeof(float) * B * h->QD,
                                hipMemcpyDeviceToDevice, s));
    HIP_TRY(h, proj(QD_PROF_O, l, part_mode));
    PROF(QD_PROF_O);
    if (tap && taps->x_mid)
      HIP_TRY(h, hipMemcpyAsync(taps->x_mid, h->x, sizeof(float) * B * H, hipMemcpyDeviceToDevice, s));
    HIP_TRY(h, proj(QD_PROF_GATE_UP, l, part_mode));
    PROF(QD_PROF_GATE_UP);
    if (tap && taps->act)
      HIP_TRY(h, hipMemcpyAsync(taps->act, h->act, sizeof(float) * B * h->I,
                                hipMemcpyDeviceToDevice, s));
    HIP_TRY(h, proj(QD_PROF_DOWN, l, part_mode));
    PROF(QD_PROF_DOWN);
    if (tap && taps->x_out)
      HIP_TRY(h, hipMemcpyAsync(taps->x_out, h->x, sizeof(float) * B * H, hipMemcpyDeviceToDevice, s));
  }
  if (taps && taps->final_h)
    HIP_TRY(h, launch_rmsnorm_rows(h->x, h->ssq, h->final_norm, H, B, h->cfg.max_batch, eps,
                                   taps->final_h, s));
  // the LM head over the leading rows: all of a decode step's, a prefill
  // chunk's first n_logits (none for a chunk that ends no prompt)
  const int B_lm = sp.n_logits < 0 ? B : sp.n_logits;
  if (B_lm > 0)
    HIP_TRY(h, launch_projection(h, B_lm, QD_PROF_LM_HEAD, 0, true, sp.logits, sp.next, s));
  PROF(QD_PROF_LM_HEAD);
#undef PROF
#ifdef QD_STEP_TRACE
  if (tracing) {
    HIP_TRY(h, hipStreamSynchronize(s));
    std::vector<unsigned long long> buf(kTraceSlots);
    FILE* f = std::fopen(std::getenv("QD_TRACE_OUT"), "wb");
    for (int c = 0; c < QD_PROF_CLASSES && f; ++c) {
      HIP_TRY(h, hipMemcpy(buf.data(), g_trace[c], kTraceSlots * 8, hipMemcpyDeviceToHost));
      std::fwrite(buf.data(), 8, kTraceSlots, f);
    }
    if (f) std::fclose(f);
  }
#endif
  return QD_OK;
}

// A decode step at batches 2-16 with the MLP half of every layer as one
// fused launch (FusedMlpArgs): embedding; per layer the QKV, attention and
// O launches of the per-stage path, then [gate/up | down]; the LM head.
// The items and split plans are those of the per-stage kernels.  Down
// writes the next layer's residual, norm sums and MFMA input pairs to the
// other buffer set (gate/up items of the same launch still read this
// one's), so the sets alternate from layer to layer; the completion
// counters alternate too (each launch clears the next one's; the embedding
// launch clears both at the start of the step).
int record_step_fused(qd_handle* h, const StepPtrs& sp, hipStream_t s) {
  const int B = sp.B, L = h->L, H = h->H, I = h->I;
  const float eps = h->cfg.rms_eps;
  const size_t layer_elems = (size_t)h->cfg.num_pages * 2 * h->Hkv * kPage * h->D;
  struct Set { float *x, *ssq; uint16_t *hi, *lo; };
  const Set set[2] = {{h->x, h->ssq, h->xg_hi, h->xg_lo}, {h->x_b, h->ssq_b, h->xg_b_hi, h->xg_b_lo}};
  const GemvPlan pq = plan_gemv(h, h->NQKV, H, B), po = plan_gemv(h, H, h->QD, B);
  const GemvPlan pd = plan_gemv(h, H, I, B), plm = plan_gemv(h, h->V, H, B, true);
  // a 128-row gate/up item yields 64 SwiGLU channels, two of down's k-tiles,
  // which must fall into one down K slice
  GemvPlan pg = plan_gemv(h, 2 * I, H, B);
  if (pg.rt == 8 && pd.kps % 2 != 0) pg = plan_gemv(h, 2 * I, H, B, false, false);
  const size_t lds_m = std::max(gemv_lds_bytes(B, pg.kps, pg.rt), gemv_lds_bytes(B, pd.kps, pd.rt));
  const int ncnt = h->fused_cnt_n / 2;  // counters per set
  unsigned* const cnt_set[2] = {h->fused_cnt, h->fused_cnt + (size_t)ncnt * kCntStride};
#ifdef QD_STEP_TRACE
  hipStreamCaptureStatus cap_st = hipStreamCaptureStatusNone;
  (void)hipStreamIsCapturing(s, &cap_st);
  const bool tracing = std::getenv("QD_TRACE_OUT") != nullptr && cap_st == hipStreamCaptureStatusNone;
  for (int c = 0; c < QD_PROF_CLASSES; ++c) {
    if (tracing && g_trace[c] == nullptr) HIP_TRY(h, hipMalloc(&g_trace[c], kTraceSlots * 8));
    if (tracing) HIP_TRY(h, hipMemsetAsync(g_trace[c], 0xff, kTraceSlots * 8, s));
  }
  auto tr = [&](int c, int l) { return tracing && l == kTraceLayer ? g_trace[c] : nullptr; };
#endif

  EmbedArgs ea{};
  ea.table = h->embed;
  ea.V = h->V; ea.H = H; ea.B = B; ea.Bmax = h->cfg.max_batch;
  ea.tokens = sp.tokens; ea.x = h->x; ea.ssq_out = h->ssq; ea.dev_flags = h->dev_flags;
  ea.xo_hi = h->xg_hi; ea.xo_lo = h->xg_lo; ea.xo_gain = h->lw[0].in_norm;
  ea.zero = h->fused_cnt; ea.nzero = 2 * ncnt;
  HIP_TRY(h, launch_embed(ea, s));

  auto gemv_args = [&](const uint16_t* w, int N, int K, const GemvPlan& p) {
    GemvArgs a{};
    a.w = w; a.N = N; a.K = K; a.B = B; a.Bmax = h->cfg.max_batch;
    a.S = p.S; a.kps = p.kps; a.rt = p.rt; a.wide = p.wide ? 1 : 0; a.eps = eps;
    return a;
  };
  // Launches that leave HBM mostly idle (attention, O, the MLP launch's
  // tail) also read the first items of the next projection into the L2 of
  // the XCD that will run each of them: attention -> O, O -> gate/up, MLP ->
  // the next QKV (or the LM head).  Batch 8 and 16: 2.98 -> 2.82 and
  // 3.54 -> 3.33 ms per step.  (The per-stage path does not: at batch 1 its
  // projections stream at full rate and the prefetch slowed the 8K step
  // from 2.85 to 2.97 ms; at 32 and 64 columns it gained nothing.)
  const int smax = attn_splits(h, B);
  for (int l = 0; l < L; ++l) {
    const LayerW& w = h->lw[l];
    const Set& P = set[l & 1];
    const Set& Q = set[(l + 1) & 1];
    GemvArgs q = gemv_args(w.qkv, h->NQKV, H, pq);
    q.x = P.x; q.xh = P.hi; q.xl = P.lo; q.ssq = P.ssq; q.gain = w.in_norm;
    q.part = h->part_qkv; q.counters = h->gemv_cnt;
#ifdef QD_STEP_TRACE
    q.trace = tr(QD_PROF_QKV, l);
#endif
    HIP_TRY(h, launch_gemv(q, kPartial, s));

    AttnArgs aa{};
    aa.qkv = h->qkv; aa.q_gain = w.q_norm; aa.k_gain = w.k_norm;
    aa.qkv_part = h->part_qkv; aa.qkv_S = pq.S; aa.qkv_rows = kTileRows * pq.rt;
    aa.rope_cos = h->rope_cos; aa.rope_sin = h->rope_sin; aa.max_pos = h->max_pos;
    aa.pool_layer = sp.pool + (size_t)l * layer_elems * h->kv_bytes;
    set_kv(h, aa);
    aa.num_pages = h->cfg.num_pages;
    aa.positions = sp.positions; aa.block_tables = sp.tables;
    aa.max_pages = h->cfg.max_pages_per_seq;
    aa.B = B; aa.Hq = h->Hq; aa.Hkv = h->Hkv;
    aa.eps = eps; aa.scale = (float)(1.0 / std::sqrt((double)h->D));
    aa.S_max = smax;
    aa.grid = attn_grid(h, B);
    aa.o_part = h->o_part; aa.ml_part = h->ml_part; aa.counters = h->attn_cnt;
    aa.out = h->attn; aa.out_hi = h->attn_hi; aa.out_lo = h->attn_lo;
    aa.dev_flags = h->dev_flags;
#ifdef QD_STEP_TRACE
    aa.trace = tr(QD_PROF_ATTN, l);
#endif
    aa.pf = next_weights(w.o, H, h->QD, po, kPrefetchWgAttn);  // O, while attention runs
    HIP_TRY(h, launch_attention(aa, h->D, h->G, kAttnWaves,
                                attn_pw(h, B), s));

    GemvArgs o = gemv_args(w.o, H, h->QD, po);  // residual in place on this set
    o.x = h->attn; o.xh = h->attn_hi; o.xl = h->attn_lo;
    o.part = h->part; o.counters = h->gemv_cnt;
    o.out = P.x; o.ssq_out = P.ssq; o.xo_hi = P.hi; o.xo_lo = P.lo; o.xo_gain = w.post_norm;
#ifdef QD_STEP_TRACE
    o.trace = tr(QD_PROF_O, l);
#endif
    o.pf = next_weights(w.gu, 2 * I, H, pg, kPrefetchWgGemv);  // the first gate/up items
    HIP_TRY(h, launch_gemv(o, kResid, s));

    FusedMlpArgs fm{};
    fm.gu = gemv_args(w.gu, 2 * I, H, pg);
    fm.gu.x = P.x; fm.gu.xh = P.hi; fm.gu.xl = P.lo; fm.gu.ssq = P.ssq; fm.gu.gain = w.post_norm;
    fm.gu.part = h->part; fm.gu.counters = h->gemv_cnt; fm.gu.out = h->act;
    fm.gu.xo_hi = h->act_hi; fm.gu.xo_lo = h->act_lo;
    fm.d = gemv_args(w.down, H, I, pd);
    fm.d.x = h->act; fm.d.xh = h->act_hi; fm.d.xl = h->act_lo;
    fm.d.part = h->part_b; fm.d.counters = h->gemv_cnt_b;
    fm.d.res_in = P.x; fm.d.out = Q.x; fm.d.ssq_out = Q.ssq; fm.d.xo_hi = Q.hi; fm.d.xo_lo = Q.lo;
    fm.d.xo_gain = l + 1 < L ? h->lw[l + 1].in_norm : h->final_norm;
    fm.ng = 2 * I / (kTileRows * pg.rt) * pg.S;
    fm.nd = H / (kTileRows * pd.rt) * pd.S;
    fm.cnt_g = cnt_set[l & 1];
    fm.cnt_other = cnt_set[(l + 1) & 1]; fm.n_other = pd.S;
    fm.dev_flags = h->dev_flags;
    fm.spin_limit = 1u << 22;
#ifdef QD_STEP_TRACE
    fm.gu.trace = tr(QD_PROF_GATE_UP, l);
    fm.d.trace = tr(QD_PROF_DOWN, l);
#endif
    // the next layer's first QKV items (after the last layer, the LM head's)
    fm.pf = l + 1 < L ? next_weights(h->lw[l + 1].qkv, h->NQKV, H, pq, kPrefetchWgGemv)
                      : next_weights(h->lm, h->V, H, plm, kPrefetchWgGemv);
    HIP_TRY(h, launch_fused_mlp(fm, lds_m, s));
  }
  // the LM head on the last layer's output set
  const Set& F = set[L & 1];
  GemvArgs lm = gemv_args(h->lm, h->V, H, plm);
  lm.x = F.x; lm.xh = F.hi; lm.xl = F.lo; lm.ssq = F.ssq; lm.gain = h->final_norm;
  lm.part = h->part; lm.counters = h->gemv_cnt;
  lm.logits = sp.logits;
  lm.amax_val = h->amax_val; lm.amax_idx = h->amax_idx; lm.amax_counter = h->amax_cnt;
  lm.amax_val2 = h->amax_val2; lm.amax_idx2 = h->amax_idx2;
  lm.next_ids = sp.next;
#ifdef QD_STEP_TRACE
  lm.trace = tracing ? g_trace[QD_PROF_LM_HEAD] : nullptr;
#endif
  HIP_TRY(h, launch_gemv(lm, kArgmax, s));
#ifdef QD_STEP_TRACE
  if (tracing) {
    HIP_TRY(h, hipStreamSynchronize(s));
    std::vector<unsigned long long> buf(kTraceSlots);
    FILE* f = std::fopen(std::getenv("QD_TRACE_OUT"), "wb");
    for (int c = 0; c < QD_PROF_CLASSES && f; ++c) {
      HIP_TRY(h, hipMemcpy(buf.data(), g_trace[c], kTraceSlots * 8, hipMemcpyDeviceToHost));
      std::fwrite(buf.data(), 8, kTraceSlots, f);
    }
    if (f) std::fclose(f);
  }
#endif
  return QD_OK;
}

// Decide whether batch 1 runs as the streaming step kernel and size it: one
// workgroup per CU (its rings take most of the LDS), each owning about
// 1/grid of every projection's row tiles.
int setup_stream(qd_handle* h) {
  // (inputs under an RMSNorm gain are the hidden size: at most 8192)
  // (the streaming kernel reads a bf16 pool only)
  if (!h->persistent || h->long_ctx || h->kv_fp8 || h->L > kStreamMaxLayers || h->H > 8192)
    return QD_OK;
  const int kmax = std::max(h->H, std::max(h->QD, h->I));
  if (kmax > 4 * 256 * kStreamStageVec) return QD_OK;  // staged input: 16 floats per thread
  auto cdiv = [](int a, int b) { return (a + b - 1) / b; };
  int W = h->num_cus;
  for (int attempt = 0; attempt < 2; ++attempt) {
    // QKV K splits (the kernel supports any count; attention sums the
    // partials).  Measured on the 4B shape, 2 splits balance the workgroups'
    // shares (3 half tiles each instead of 1 or 2 tiles) but lose more to the
    // shorter runs, the extra epilogues and attention's extra input loads
    // (2.44 and, with 4 splits, 2.51 ms per step against 2.37): one split.
    const int Rq = h->NQKV / kTileRows;
    const int qS = 1;
    const int rt_max = std::max(cdiv(Rq * qS, W),
                                std::max(cdiv(h->H / kTileRows, W), cdiv(2 * h->I / kTileRows, W)));
    // inputs are staged in whole KB (256 floats), the old residual rows after them
    const int res_off = cdiv(kmax, 256) * 256;
    const int in_floats = res_off + cdiv(h->H / kTileRows, W) * kTileRows;
    const size_t lds = stream_lds_bytes(h->D, h->G, in_floats, rt_max);
    if (lds == 0) return QD_OK;
    int g = 0;
    if (stream_max_grid(h->D, h->G, lds, h->num_cus, &g) != hipSuccess || g < 1) {
      (void)hipGetLastError();  // LDS beyond the device limit: no streaming step
      return QD_OK;
    }
    if (g >= W) {
      // the waves' tile runs, from the same partition the kernel consumes
      StreamArgs sa{};
      sa.L = h->L; sa.H = h->H; sa.QD = h->QD; sa.I = h->I; sa.V = h->V; sa.NQKV = h->NQKV;
      sa.qkv_S = qS;
      for (int l = 0; l < h->L; ++l) {
        const LayerW& w = h->lw[l];
        sa.w[4 * l + 0] = w.qkv; sa.w[4 * l + 1] = w.o; sa.w[4 * l + 2] = w.gu; sa.w[4 * l + 3] = w.down;
      }
      sa.lm = h->lm;
      std::vector<StreamRun> runs;
      std::vector<int> off((size_t)W * 4);
      for (int wg = 0; wg < W; ++wg)
        for (int wave = 0; wave < 4; ++wave) {
          off[(size_t)wg * 4 + wave] = (int)runs.size();
          stream_runs(sa, W, wg, wave, [&](const unsigned char* p, int n, int stride, int u) {
            runs.push_back(StreamRun{p, (uint32_t)n | ((uint32_t)u << 16), (uint32_t)stride});
          });
        }
      int rc = dev_alloc(h, &h->stream_runs, runs.size());
      if (!rc) rc = dev_alloc(h, &h->stream_run_off, off.size());
      if (rc) return rc;
      HIP_TRY(h, hipMemcpy(h->stream_runs, runs.data(), runs.size() * sizeof(StreamRun),
                           hipMemcpyHostToDevice));
      HIP_TRY(h, hipMemcpy(h->stream_run_off, off.data(), off.size() * sizeof(int),
                           hipMemcpyHostToDevice));
      h->stream_ok = true;
      h->stream_grid = W;
      h->stream_lds = lds;
      h->stream_in_floats = in_floats;
      h->stream_res_off = res_off;
      h->stream_rt_max = rt_max;
      h->stream_qkv_S = qS;
      return QD_OK;
    }
    W = g;
  }
  return QD_OK;
}

// One batch-1 step as the streaming cooperative kernel (taps: copy one
// layer's intermediates out, for checking; may be null).
int run_stream(qd_handle* h, const StepPtrs& sp, hipStream_t s, const qd_taps* taps = nullptr) {
  const int H = h->H;
  StreamArgs a{};
  a.embed.table = h->embed;
  a.embed.V = h->V; a.embed.H = H; a.embed.B = 1; a.embed.Bmax = h->cfg.max_batch;
  a.embed.tokens = sp.tokens; a.embed.x = h->x; a.embed.ssq_out = h->ssq;
  a.embed.dev_flags = h->dev_flags;
  AttnArgs& at = a.attn;
  at.qkv = h->qkv;
  at.qkv_part = h->part_qkv;
  at.qkv_S = h->stream_qkv_S;
  at.qkv_rows = kTileRows;
  at.rope_cos = h->rope_cos; at.rope_sin = h->rope_sin; at.max_pos = h->max_pos;
  at.pool_layer = sp.pool;
  set_kv(h, at);
  at.num_pages = h->cfg.num_pages;
  at.positions = sp.positions; at.block_tables = sp.tables;
  at.max_pages = h->cfg.max_pages_per_seq;
  at.B = 1; at.Hq = h->Hq; at.Hkv = h->Hkv;
  at.eps = h->cfg.rms_eps; at.scale = (float)(1.0 / std::sqrt((double)h->D));
  at.S_max = stream_attn_splits(h);
  at.o_part = h->o_part; at.ml_part = h->ml_part; at.counters = h->attn_cnt;
  at.out = h->attn;
  at.dev_flags = h->dev_flags;
  a.layers = h->layers_dev;
  for (int l = 0; l < h->L; ++l) {
    const LayerW& w = h->lw[l];
    a.w[4 * l + 0] = w.qkv; a.w[4 * l + 1] = w.o; a.w[4 * l + 2] = w.gu; a.w[4 * l + 3] = w.down;
  }
  a.L = h->L; a.H = H; a.QD = h->QD; a.I = h->I; a.V = h->V; a.NQKV = h->NQKV;
  a.Bmax = h->cfg.max_batch;
  a.lm = h->lm; a.final_norm = h->final_norm; a.eps = h->cfg.rms_eps;
  a.x = h->x; a.ssq = h->ssq; a.qkv = h->qkv; a.attn_out = h->attn; a.act = h->act;
  a.logits = sp.logits;
  a.amax_val = h->stream_amax_val; a.amax_idx = h->stream_amax_idx;
  a.next_ids = sp.next;
  a.pool_layer_elems = (size_t)h->cfg.num_pages * 2 * h->Hkv * kPage * h->D;
  a.runs = h->stream_runs;
  a.run_off = h->stream_run_off;
  a.qkv_S = h->stream_qkv_S;
  a.qkv_part = h->part_qkv;
  a.in_floats = h->stream_in_floats;
  a.res_off = h->stream_res_off;
  a.rt_max = h->stream_rt_max;
  a.cnt = h->step_cnt; a.flags = h->step_flags;
  a.exit_cnt = h->step_exit; a.abort_flag = h->step_abort;
  a.dev_flags = h->dev_flags;
  a.spin_limit = 1u << 22;  // polls; a few seconds, far beyond any real wait
  a.tap_layer = -1;
  a.attn_tap = a.attn;
  if (taps != nullptr) {
    a.tap_layer = taps->layer;
    a.tap_x_in = taps->x_in; a.tap_qkv = taps->qkv; a.tap_attn = taps->attn;
    a.tap_x_mid = taps->x_mid; a.tap_act = taps->act; a.tap_x_out = taps->x_out;
    a.tap_final_h = taps->final_h;
    a.attn_tap.tap_q = taps->q_rot;
    a.attn_tap.tap_k = taps->k_rot;
  }
#ifdef QD_STEP_TRACE
  static unsigned long long* trace = nullptr;
  const size_t trace_n = (size_t)h->stream_grid * 1024 * 3;
  if (!trace) {
    HIP_TRY(h, hipMalloc(&trace, trace_n * 8));
  }
  HIP_TRY(h, hipMemsetAsync(trace, 0xff, trace_n * 8, s));
  a.trace = trace;
#endif
  HIP_TRY(h, launch_stream(a, h->D, h->G, h->stream_grid, h->stream_lds, s));
#ifdef QD_STEP_TRACE
  if (const char* path = std::getenv("QD_TRACE_OUT")) {
    HIP_TRY(h, hipStreamSynchronize(s));
    std::vector<unsigned long long> hostbuf(trace_n);
    HIP_TRY(h, hipMemcpy(hostbuf.data(), trace, trace_n * 8, hipMemcpyDeviceToHost));
    FILE* f = std::fopen(path, "wb");
    if (f) {
      std::fwrite(hostbuf.data(), 8, trace_n, f);
      std::fclose(f);
    }
  }
#endif
  return QD_OK;
}

bool all_loaded(const qd_handle* h, std::string* missing) {
  for (auto& kv : h->expected)
    if (!kv.second) { *missing = kv.first; return false; }
  return true;
}

int check_step_args(qd_handle* h, int32_t batch, const void* a, const void* b, const void* c,
                    const void* d, const void* e) {
  if (!h) return QD_EINVAL;
  if (batch < 1 || batch > h->cfg.max_batch) return fail(h, QD_EINVAL, "batch out of range");
  if (!a || !b || !c || !d || !e) return fail(h, QD_EINVAL, "NULL step pointer");
  std::string missing;
  if (!all_loaded(h, &missing)) return fail(h, QD_ESTATE, "weight not loaded: " + missing);
  return QD_OK;
}

// GEMM workgroup tile (weight rows x input rows) of an N-row projection
// over M input rows: 128x128 when those tiles give between half a CU's and
// one CU's worth of workgroups (one round, each workgroup on a CU of its
// own), else 128x64, and 64x64 only when 128x64 tiles would leave three
// quarters of the CUs idle.  On a 512-row Qwen3-4B prompt this picks
// 128x128 for QKV and 128x64 for O, gate/up and down: a sweep of the four
// shapes per projection measured these fastest (O and down 64x64: +0.2 and
// +0.7 ms per prompt; gate/up 128x128: +0.1 ms; QKV 128x64: +0.1 ms).
void pf_tile(const qd_handle* h, int N, int M, int* wn, int* wm) {
  auto tiles = [&](int a, int b) {
    return (long long)((N + 32 * a - 1) / (32 * a)) * ((M + 32 * b - 1) / (32 * b));
  };
  if (2 * tiles(4, 4) >= h->num_cus && tiles(4, 4) <= h->num_cus) {
    *wn = 4; *wm = 4;
  } else if (4 * tiles(4, 2) >= h->num_cus) {
    *wn = 4; *wm = 2;
  } else {
    *wn = 2; *wm = 2;
  }
}

hipError_t pf_gemm(qd_handle* h, int mode, const uint16_t* w, int N, int K, const uint16_t* x,
                   int M, float* out, int ldo, uint16_t* act, hipStream_t s) {
  int wn = 4, wm = 4;
  pf_tile(h, N, M, &wn, &wm);
  PfGemmArgs a{};
  a.w = w; a.x = x; a.N = N; a.K = K; a.M = M;
  a.nb_n = (N + 32 * wn - 1) / (32 * wn);
  a.nb_m = (M + 32 * wm - 1) / (32 * wm);
  a.out = out; a.ldo = ldo; a.act = act;
  return launch_pf_gemm(a, mode, wn, wm, s);
}

// Enqueue a prompt chunk (qd_prefill_prompts) on the handle's stream.
int record_prefill_prompts(qd_handle* h, const PfSegs& sg, const int32_t* tokens,
                           const int32_t* tables, unsigned char* pool, int n_logits, int32_t* next,
                           float* logits) {
  hipStream_t s = h->stream;
  const int L = h->L, H = h->H, I = h->I, M = sg.row0[sg.n];
  const int Mt = (M + 15) / 16 * 16;
  const float eps = h->cfg.rms_eps;
  const size_t layer_elems = (size_t)h->cfg.num_pages * 2 * h->Hkv * kPage * h->D;
  HIP_TRY(h, launch_pf_embed(h->embed, h->V, H, tokens, M, h->pf_x, h->dev_flags, s));
  PfAttnArgs aa{};
  aa.qkv = h->pf_qkv;
  aa.rope_cos = h->rope_cos; aa.rope_sin = h->rope_sin;
  aa.num_pages = h->cfg.num_pages;
  aa.kv_fp8 = h->kv_fp8 ? 1 : 0;
  aa.k_scale = h->k_scale; aa.v_scale = h->v_scale;
  aa.k_inv = 1.f / h->k_scale; aa.v_inv = 1.f / h->v_scale;
  aa.block_tables = tables; aa.max_pages = h->cfg.max_pages_per_seq;
  aa.M = M; aa.Hq = h->Hq; aa.Hkv = h->Hkv;
  aa.eps = eps; aa.scale = (float)(1.0 / std::sqrt((double)h->D));
  aa.q_hi = h->pf_q_hi; aa.q_lo = h->pf_q_lo;
  aa.out = h->pf_tin;
  aa.dev_flags = h->dev_flags;
  aa.seg = sg;
  for (int l = 0; l < L; ++l) {
    const LayerW& w = h->lw[l];
    HIP_TRY(h, launch_pf_norm(h->pf_x, w.in_norm, H, M, Mt, eps, h->pf_tin, s));
    HIP_TRY(h, pf_gemm(h, kPfStore, w.qkv, h->NQKV, H, h->pf_tin, M, h->pf_qkv, h->NQKV, nullptr, s));
    aa.q_gain = w.q_norm; aa.k_gain = w.k_norm;
    aa.pool_layer = pool + (size_t)l * layer_elems * h->kv_bytes;
    HIP_TRY(h, launch_pf_qk(aa, h->D, s));
    HIP_TRY(h, launch_pf_attn(aa, h->D, h->G, s));
    HIP_TRY(h, pf_gemm(h, kPfResid, w.o, H, h->QD, h->pf_tin, M, h->pf_x, H, nullptr, s));
    HIP_TRY(h, launch_pf_norm(h->pf_x, w.post_norm, H, M, Mt, eps, h->pf_tin, s));
    HIP_TRY(h, pf_gemm(h, kPfSwiGLU, w.gu, 2 * I, H, h->pf_tin, M, nullptr, 0, h->pf_tact, s));
    HIP_TRY(h, pf_gemm(h, kPfResid, w.down, H, I, h->pf_tact, M, h->pf_x, H, nullptr, s));
  }
  if (n_logits > 0) {
    // each segment's last row, in the decode step's buffers, then the step's LM head
    const bool mfma = gemv_mfma(n_logits);
    HIP_TRY(h, launch_pf_head_rows(h->pf_x, H, sg, n_logits, h->final_norm, h->x, h->ssq,
                                   h->cfg.max_batch, mfma ? h->xg_hi : nullptr,
                                   mfma ? h->xg_lo : nullptr, s));
    HIP_TRY(h, launch_projection(h, n_logits, QD_PROF_LM_HEAD, 0, true, logits, next, s));
  }
  return QD_OK;
}

}  // namespace

int qd::set_global_error(int code, const std::string& msg) {
  g_create_error = msg;
  return code;
}

const qd_config* qd::handle_config(const qd_handle* h) { return &h->cfg; }

int qd::handle_fail(qd_handle* h, int code, const std::string& msg) { return fail(h, code, msg); }

extern "C" {

int qd_create(const qd_config* cfg, void* hip_stream, qd_handle** out) {
  if (!out) return fail(nullptr, QD_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = validate_config(cfg);
  if (rc) return rc;
  qd_handle* h = new qd_handle();
  h->cfg = *cfg;
  h->stream = static_cast<hipStream_t>(hip_stream);
  h->L = cfg->num_layers; h->H = cfg->hidden; h->Hq = cfg->num_q_heads;
  h->Hkv = cfg->num_kv_heads; h->D = cfg->head_dim; h->I = cfg->intermediate;
  h->V = cfg->vocab; h->QD = h->Hq * h->D; h->KD = h->Hkv * h->D;
  h->NQKV = h->QD + 2 * h->KD; h->G = h->Hq / h->Hkv;
  h->kv_fp8 = cfg->kv_dtype == 1;
  h->kv_bytes = h->kv_fp8 ? 1 : 2;
  if (h->kv_fp8) { h->k_scale = cfg->k_scale; h->v_scale = cfg->v_scale; }

  auto bail = [&](int code) {
    g_create_error = h->err;
    qd_destroy(h);
    return code;
  };
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) { hip_fail(h, e, "hipGetDevice"); return bail(QD_EHIP); }
  e = hipDeviceGetAttribute(&h->num_cus, hipDeviceAttributeMultiprocessorCount, h->device);
  if (e != hipSuccess) { hip_fail(h, e, "hipDeviceGetAttribute"); return bail(QD_EHIP); }
  e = hipStreamCreateWithFlags(&h->cap, hipStreamNonBlocking);
  if (e != hipSuccess) { hip_fail(h, e, "hipStreamCreate"); return bail(QD_EHIP); }

  const int L = h->L, H = h->H, I = h->I, V = h->V, Bm = cfg->max_batch;
  // packed weights
  h->lw.resize(L);
  for (int l = 0; l < L; ++l) {
    LayerW& w = h->lw[l];
    if ((rc = dev_alloc(h, &w.qkv, (size_t)h->NQKV * H))) return bail(rc);
    if ((rc = dev_alloc(h, &w.o, (size_t)H * h->QD))) return bail(rc);
    if ((rc = dev_alloc(h, &w.gu, (size_t)2 * I * H))) return bail(rc);
    if ((rc = dev_alloc(h, &w.down, (size_t)H * I))) return bail(rc);
    if ((rc = dev_alloc(h, &w.in_norm, H))) return bail(rc);
    if ((rc = dev_alloc(h, &w.post_norm, H))) return bail(rc);
    if ((rc = dev_alloc(h, &w.q_norm, h->D))) return bail(rc);
    if ((rc = dev_alloc(h, &w.k_norm, h->D))) return bail(rc);
    const std::string p = "model.layers." + std::to_string(l) + ".";
    for (const char* n : {"input_layernorm", "self_attn.q_proj", "self_attn.k_proj",
                          "self_attn.v_proj", "self_attn.o_proj", "self_attn.q_norm",
                          "self_attn.k_norm", "post_attention_layernorm", "mlp.gate_proj",
                          "mlp.up_proj", "mlp.down_proj"})
      h->expected[p + n + ".weight"] = 0;
  }
  if ((rc = dev_alloc(h, &h->embed, (size_t)V * H))) return bail(rc);
  if (cfg->tie_embeddings) {
    h->lm = h->embed;
  } else {
    if ((rc = dev_alloc(h, &h->lm, (size_t)V * H))) return bail(rc);
    h->expected["lm_head.weight"] = 0;
  }
  if ((rc = dev_alloc(h, &h->final_norm, H))) return bail(rc);
  h->expected["model.embed_tokens.weight"] = 0;
  h->expected["model.norm.weight"] = 0;

  h->persistent = cfg->persistent != 0;
  h->long_ctx = cfg->max_pages_per_seq > kStreamMaxPages;
  h->mid_ctx = cfg->max_pages_per_seq >= kMidCtxPages;
  if ((rc = setup_stream(h))) return bail(rc);

  // activations and scratch
  if ((rc = dev_alloc(h, &h->x, (size_t)Bm * H))) return bail(rc);
  if ((rc = dev_alloc(h, &h->ssq, (size_t)(H / kSsqRows) * Bm))) return bail(rc);
  if ((rc = dev_alloc(h, &h->qkv, (size_t)Bm * h->NQKV))) return bail(rc);
  if ((rc = dev_alloc(h, &h->attn, (size_t)Bm * h->QD))) return bail(rc);
  if ((rc = dev_alloc(h, &h->act, (size_t)Bm * I))) return bail(rc);
  if (gemv_mfma(Bm)) {
    // MFMA operands cover whole blocks of 8 or 16 batch columns: rows up to
    // the block are allocated and zeroed (rows >= B only feed unused outputs)
    const size_t rows = (size_t)gemv_nb(Bm);
    uint16_t** bufs[8] = {&h->xg_hi, &h->xg_lo, &h->attn_hi, &h->attn_lo, &h->act_hi, &h->act_lo,
                          &h->xg_b_hi, &h->xg_b_lo};
    const size_t cols[8] = {(size_t)H, (size_t)H, (size_t)h->QD, (size_t)h->QD, (size_t)I, (size_t)I,
                            (size_t)H, (size_t)H};
    for (int i = 0; i < 8; ++i) {
      if ((rc = dev_alloc(h, bufs[i], rows * cols[i]))) return bail(rc);
      e = hipMemset(*bufs[i], 0, rows * cols[i] * sizeof(uint16_t));
      if (e != hipSuccess) { hip_fail(h, e, "hipMemset"); return bail(QD_EHIP); }
    }
  }
  // split partials: N * S * B floats for whichever projection needs most;
  // arrival counters: one per row group, at most N / 16
  size_t part_elems = 1, part_qkv_elems = 1;
  const int max_nrg = std::max(std::max(h->NQKV, 2 * I), std::max(H, V)) / kTileRows;
  for (int B = 1; B <= Bm; ++B) {
    // the same plans the steps will use
    const int dims[3][2] = {{H, h->QD}, {H, I}, {2 * I, H}};
    for (auto& d : dims) {
      GemvPlan p = plan_gemv(h, d[0], d[1], B);
      if (p.S > 1) part_elems = std::max(part_elems, (size_t)d[0] * p.S * B);
    }
    const GemvPlan pl = plan_gemv(h, V, H, B, true);
    if (pl.S > 1) part_elems = std::max(part_elems, (size_t)V * pl.S * B);
    const GemvPlan pq = plan_gemv(h, h->NQKV, H, B);
    part_qkv_elems = std::max(part_qkv_elems, (size_t)h->NQKV * pq.S * B);
  }
  if ((rc = dev_alloc(h, &h->part, part_elems))) return bail(rc);
  if (h->stream_ok) part_qkv_elems = std::max(part_qkv_elems, (size_t)h->NQKV * h->stream_qkv_S);
  if ((rc = dev_alloc(h, &h->part_qkv, part_qkv_elems))) return bail(rc);
  if ((rc = dev_alloc(h, &h->gemv_cnt, (size_t)max_nrg * kCntStride))) return bail(rc);
  // fused launches (see record_step_fused)
  if ((rc = dev_alloc(h, &h->x_b, (size_t)Bm * H))) return bail(rc);
  if ((rc = dev_alloc(h, &h->ssq_b, (size_t)(H / kSsqRows) * Bm))) return bail(rc);
  if ((rc = dev_alloc(h, &h->part_b, part_elems))) return bail(rc);
  if ((rc = dev_alloc(h, &h->gemv_cnt_b, (size_t)max_nrg * kCntStride))) return bail(rc);
  {
    int max_down_splits = 1;
    for (int B = 1; B <= Bm; ++B) max_down_splits = std::max(max_down_splits, plan_gemv(h, H, I, B).S);
    h->fused_cnt_n = 2 * max_down_splits;  // two alternating sets
    if ((rc = dev_alloc(h, &h->fused_cnt, (size_t)h->fused_cnt_n * kCntStride))) return bail(rc);
    e = hipMemset(h->fused_cnt, 0, sizeof(unsigned) * h->fused_cnt_n * kCntStride);
    if (e == hipSuccess)
      e = hipMemset(h->gemv_cnt_b, 0, sizeof(unsigned) * max_nrg * kCntStride);
    if (e != hipSuccess) { hip_fail(h, e, "hipMemset"); return bail(QD_EHIP); }
  }
  size_t att_rows = 0;
  for (int B = 1; B <= Bm; ++B)
    att_rows = std::max(att_rows, (size_t)B * h->Hq * attn_splits(h, B));
  if (h->stream_ok) att_rows = std::max(att_rows, (size_t)h->Hq * stream_attn_splits(h));
  if ((rc = dev_alloc(h, &h->o_part, att_rows * h->D))) return bail(rc);
  if ((rc = dev_alloc(h, &h->ml_part, att_rows * 2))) return bail(rc);
  if ((rc = dev_alloc(h, &h->attn_cnt, (size_t)Bm * h->Hkv * kCntStride))) return bail(rc);
  const size_t nrg_v = V / kRowsPerGroup, ng2_v = (nrg_v + 63) / 64;
  if ((rc = dev_alloc(h, &h->amax_val, nrg_v * Bm))) return bail(rc);
  if ((rc = dev_alloc(h, &h->amax_idx, nrg_v * Bm))) return bail(rc);
  if ((rc = dev_alloc(h, &h->amax_val2, ng2_v * Bm))) return bail(rc);
  if ((rc = dev_alloc(h, &h->amax_idx2, ng2_v * Bm))) return bail(rc);
  if ((rc = dev_alloc(h, &h->amax_cnt, (ng2_v + 1) * kCntStride))) return bail(rc);
  if ((rc = dev_alloc(h, &h->dev_flags, 1))) return bail(rc);
  if ((rc = dev_alloc(h, &h->prof_ids, (size_t)Bm))) return bail(rc);
  sample_split(V, &h->sample_G, &h->sample_C);
  if (h->sample_G > kMaxSampleChunks ||
      (size_t)h->sample_G * 512 > (size_t)h->sample_C * 4)  // the merge reuses the chunk's LDS
  {
    fail(h, QD_EUNSUPPORTED, "vocab too large for on-device sampling (at most 524288)");
    return bail(QD_EUNSUPPORTED);
  }
  {
    const size_t slots = (size_t)Bm * h->sample_G;
    if ((rc = dev_alloc(h, &h->sample_max, slots))) return bail(rc);
    if ((rc = dev_alloc(h, &h->sample_idx, slots))) return bail(rc);
    if ((rc = dev_alloc(h, &h->sample_cand, slots * 64))) return bail(rc);
    if ((rc = dev_alloc(h, &h->sample_cnt, (size_t)Bm * kCntStride))) return bail(rc);
    if ((rc = dev_alloc(h, &h->sample_sum, slots))) return bail(rc);
    if ((rc = dev_alloc(h, &h->sample_cnt2, (size_t)Bm * kCntStride))) return bail(rc);
    if ((rc = dev_alloc(h, &h->sample_hist, (size_t)Bm * 256))) return bail(rc);
    if ((rc = dev_alloc(h, &h->sample_pass_hist, (size_t)Bm * kPassHists * 256))) return bail(rc);
    if ((rc = dev_alloc(h, &h->sample_sum2, slots))) return bail(rc);
    if ((rc = dev_alloc(h, &h->sample_sum3, slots))) return bail(rc);
    if ((rc = dev_alloc(h, &h->sample_cnt3, (size_t)Bm * kCntStride))) return bail(rc);
    if ((rc = dev_alloc(h, &h->sample_flag, (size_t)Bm))) return bail(rc);
    if ((rc = dev_alloc(h, &h->sample_cut, (size_t)Bm * 2))) return bail(rc);
    e = hipMemset(h->sample_cnt, 0, sizeof(unsigned) * Bm * kCntStride);
    if (e == hipSuccess) e = hipMemset(h->sample_cnt2, 0, sizeof(unsigned) * Bm * kCntStride);
    if (e == hipSuccess) e = hipMemset(h->sample_hist, 0, sizeof(double) * Bm * 256);
    if (e == hipSuccess) e = hipMemset(h->sample_pass_hist, 0, sizeof(double) * Bm * kPassHists * 256);
    if (e == hipSuccess) e = hipMemset(h->sample_cnt3, 0, sizeof(unsigned) * Bm * kCntStride);
    if (e == hipSuccess) e = hipMemset(h->sample_flag, 0, sizeof(int) * Bm);
    if (e != hipSuccess) { hip_fail(h, e, "hipMemset"); return bail(QD_EHIP); }
  }
  e = hipMemset(h->gemv_cnt, 0, sizeof(unsigned) * max_nrg * kCntStride);
  if (e == hipSuccess) e = hipMemset(h->attn_cnt, 0, sizeof(unsigned) * Bm * h->Hkv * kCntStride);
  if (e == hipSuccess) e = hipMemset(h->amax_cnt, 0, sizeof(unsigned) * (ng2_v + 1) * kCntStride);
  if (e == hipSuccess) e = hipMemset(h->dev_flags, 0, sizeof(int));
  if (e != hipSuccess) { hip_fail(h, e, "hipMemset"); return bail(QD_EHIP); }

  // streaming step state
  if (h->stream_ok) {
    if ((rc = dev_alloc(h, &h->layers_dev, (size_t)L))) return bail(rc);
    // (the streaming step also counts the LM head's workgroups)
    if ((rc = dev_alloc(h, &h->step_cnt, (size_t)2 + (size_t)L * kCntPerLayer))) return bail(rc);
    if ((rc = dev_alloc(h, &h->step_flags, (size_t)2 * h->num_cus * 32))) return bail(rc);
    if ((rc = dev_alloc(h, &h->step_exit, 1))) return bail(rc);
    if ((rc = dev_alloc(h, &h->step_abort, 1))) return bail(rc);
    if ((rc = dev_alloc(h, &h->stream_amax_val, (size_t)h->stream_grid))) return bail(rc);
    if ((rc = dev_alloc(h, &h->stream_amax_idx, (size_t)h->stream_grid))) return bail(rc);
    e = hipMemset(h->step_cnt, 0, sizeof(unsigned) * (2 + (size_t)L * kCntPerLayer));
    if (e == hipSuccess) e = hipMemset(h->step_flags, 0, sizeof(unsigned) * 2 * h->num_cus * 32);
    if (e == hipSuccess) e = hipMemset(h->step_exit, 0, sizeof(unsigned));
    if (e == hipSuccess) e = hipMemset(h->step_abort, 0, sizeof(unsigned));
    std::vector<LayerDev> ld(L);
    for (int l = 0; l < L; ++l) {
      const LayerW& w = h->lw[l];
      ld[l] = LayerDev{w.qkv, w.o, w.gu, w.down, w.in_norm, w.post_norm, w.q_norm, w.k_norm};
    }
    if (e == hipSuccess)
      e = hipMemcpy(h->layers_dev, ld.data(), sizeof(LayerDev) * L, hipMemcpyHostToDevice);
    if (e != hipSuccess) { hip_fail(h, e, "persistent state"); return bail(QD_EHIP); }
  }

  // prompt-chunk workspace, zeroed once (operand-tile rows past a chunk's
  // last are read by the GEMMs and must hold finite values)
  if (cfg->max_prefill_rows > 0) {
    const size_t Mp = (size_t)((cfg->max_prefill_rows + kPfRowAlign - 1) / kPfRowAlign) * kPfRowAlign;
    h->pf_rows = (int)Mp;
    const size_t tin = Mp * std::max(H, h->QD) * 2, tact = Mp * I * 2;
    if ((rc = dev_alloc(h, &h->pf_x, Mp * H))) return bail(rc);
    if ((rc = dev_alloc(h, &h->pf_qkv, Mp * h->NQKV))) return bail(rc);
    if ((rc = dev_alloc(h, &h->pf_q_hi, Mp * h->QD))) return bail(rc);
    if ((rc = dev_alloc(h, &h->pf_q_lo, Mp * h->QD))) return bail(rc);
    if ((rc = dev_alloc(h, &h->pf_tin, tin))) return bail(rc);
    if ((rc = dev_alloc(h, &h->pf_tact, tact))) return bail(rc);
    e = hipMemset(h->pf_tin, 0, tin * sizeof(uint16_t));
    if (e == hipSuccess) e = hipMemset(h->pf_tact, 0, tact * sizeof(uint16_t));
    if (e != hipSuccess) { hip_fail(h, e, "hipMemset"); return bail(QD_EHIP); }
  }

  // RoPE table: angle p * theta^(-2i/D) in double, cos/sin rounded once to fp32.
  h->max_pos = cfg->max_pages_per_seq * kPage;
  const int half = h->D / 2;
  std::vector<float> cs((size_t)h->max_pos * half), sn((size_t)h->max_pos * half);
  for (int i = 0; i < half; ++i) {
    const double inv_freq = std::pow(cfg->rope_theta, -2.0 * i / h->D);
    for (int p = 0; p < h->max_pos; ++p) {
      const double a = (double)p * inv_freq;
      cs[(size_t)p * half + i] = (float)std::cos(a);
      sn[(size_t)p * half + i] = (float)std::sin(a);
    }
  }
  if ((rc = dev_alloc(h, &h->rope_cos, cs.size()))) return bail(rc);
  if ((rc = dev_alloc(h, &h->rope_sin, sn.size()))) return bail(rc);
  e = hipMemcpy(h->rope_cos, cs.data(), cs.size() * sizeof(float), hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(h->rope_sin, sn.data(), sn.size() * sizeof(float), hipMemcpyHostToDevice);
  if (e != hipSuccess) { hip_fail(h, e, "hipMemcpy"); return bail(QD_EHIP); }
  *out = h;
  return QD_OK;
}

int qd_load_weights(qd_handle* h, const qd_tensor_desc* t, int32_t n) {
  if (!h) return QD_EINVAL;
  if (n < 0 || (n > 0 && !t)) return fail(h, QD_EINVAL, "bad tensor list");
  const int H = h->H, I = h->I, V = h->V, D = h->D;
  hipStream_t s = h->stream;
  for (int i = 0; i < n; ++i) {
    const qd_tensor_desc& d = t[i];
    if (!d.name || !d.data) return fail(h, QD_EINVAL, "tensor with NULL name or data");
    const std::string name = d.name;
    auto it = h->expected.find(name);
    if (it == h->expected.end()) return fail(h, QD_EINVAL, "unexpected tensor " + name);
    if (d.dtype != 0) return fail(h, QD_EINVAL, "tensor " + name + " is not bf16");
    auto need = [&](int64_t r, int64_t c) {
      if (c < 0) return d.ndim == 1 && d.shape[0] == r;
      return d.ndim == 2 && d.shape[0] == r && d.shape[1] == c;
    };
    const uint16_t* src = static_cast<const uint16_t*>(d.data);
    hipError_t e = hipSuccess;
    bool shape_ok = true;
    if (name == "model.embed_tokens.weight") {
      shape_ok = need(V, H);
      if (shape_ok) e = launch_repack(src, V, H, h->embed, 16, 16, 0, s);
    } else if (name == "lm_head.weight") {
      shape_ok = need(V, H);
      if (shape_ok) e = launch_repack(src, V, H, h->lm, 16, 16, 0, s);
    } else if (name == "model.norm.weight") {
      shape_ok = need(H, -1);
      if (shape_ok) e = launch_bf16_to_f32(src, h->final_norm, H, s);
    } else {
      const int l = std::atoi(name.c_str() + std::strlen("model.layers."));
      LayerW& w = h->lw[l];
      const std::string leaf = name.substr(name.find('.', std::strlen("model.layers.")) + 1);
      if (leaf == "input_layernorm.weight") {
        shape_ok = need(H, -1);
        if (shape_ok) e = launch_bf16_to_f32(src, w.in_norm, H, s);
      } else if (leaf == "post_attention_layernorm.weight") {
        shape_ok = need(H, -1);
        if (shape_ok) e = launch_bf16_to_f32(src, w.post_norm, H, s);
      } else if (leaf == "self_attn.q_norm.weight") {
        shape_ok = need(D, -1);
        if (shape_ok) e = launch_bf16_to_f32(src, w.q_norm, D, s);
      } else if (leaf == "self_attn.k_norm.weight") {
        shape_ok = need(D, -1);
        if (shape_ok) e = launch_bf16_to_f32(src, w.k_norm, D, s);
      } else if (leaf == "self_attn.q_proj.weight") {
        shape_ok = need(h->QD, H);
        if (shape_ok) e = launch_repack(src, h->QD, H, w.qkv, 16, 16, 0, s);
      } else if (leaf == "self_attn.k_proj.weight") {
        shape_ok = need(h->KD, H);
        if (shape_ok) e = launch_repack(src, h->KD, H, w.qkv, 16, 16, h->QD, s);
      } else if (leaf == "self_attn.v_proj.weight") {
        shape_ok = need(h->KD, H);
        if (shape_ok) e = launch_repack(src, h->KD, H, w.qkv, 16, 16, h->QD + h->KD, s);
      } else if (leaf == "self_attn.o_proj.weight") {
        shape_ok = need(H, h->QD);
        if (shape_ok) e = launch_repack(src, H, h->QD, w.o, 16, 16, 0, s);
      } else if (leaf == "mlp.gate_proj.weight") {
        shape_ok = need(I, H);
        if (shape_ok) e = launch_repack(src, I, H, w.gu, 8, 16, 0, s);
      } else if (leaf == "mlp.up_proj.weight") {
        shape_ok = need(I, H);
        if (shape_ok) e = launch_repack(src, I, H, w.gu, 8, 16, 8, s);
      } else if (leaf == "mlp.down_proj.weight") {
        shape_ok = need(H, I);
        if (shape_ok) e = launch_repack(src, H, I, w.down, 16, 16, 0, s);
      } else {
        return fail(h, QD_EINVAL, "unexpected tensor " + name);
      }
    }
    if (!shape_ok) return fail(h, QD_EINVAL, "tensor " + name + " has the wrong shape");
    if (e != hipSuccess) return hip_fail(h, e, "repack launch");
    it->second = 1;
  }
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(h, e, "hipStreamSynchronize");
  // weights changed: captured graphs stay valid (same addresses)
  return QD_OK;
}

int qd_decode_step_taps(qd_handle* h, int32_t batch, const int32_t* token_ids,
                        const int32_t* positions, const int32_t* block_tables, void* kv_pool,
                        int32_t* out_next_ids, float* out_logits, const qd_taps* taps) {
  int rc = check_step_args(h, batch, token_ids, positions, block_tables, kv_pool, out_next_ids);
  if (rc) return rc;
  StepPtrs sp{batch, token_ids, positions, block_tables, static_cast<unsigned char*>(kv_pool),
              out_next_ids, out_logits};
  return record_step(h, sp, taps, h->stream);
}

int qd_stream_step_taps(qd_handle* h, const int32_t* token_ids, const int32_t* positions,
                        const int32_t* block_tables, void* kv_pool, int32_t* out_next_ids,
                        float* out_logits, const qd_taps* taps) {
  int rc = check_step_args(h, 1, token_ids, positions, block_tables, kv_pool, out_next_ids);
  if (rc) return rc;
  if (!use_stream(h, 1))
    return fail(h, QD_EUNSUPPORTED, "this handle does not run batch 1 as the streaming kernel");
  StepPtrs sp{1, token_ids, positions, block_tables, static_cast<unsigned char*>(kv_pool),
              out_next_ids, out_logits};
  return run_stream(h, sp, h->stream, taps);
}

int qd_decode_step(qd_handle* h, int32_t batch, const int32_t* token_ids,
                   const int32_t* positions, const int32_t* block_tables, void* kv_pool,
                   int32_t* out_next_ids, float* out_logits) {
  int rc = check_step_args(h, batch, token_ids, positions, block_tables, kv_pool, out_next_ids);
  if (rc) return rc;
  StepPtrs sp{batch, token_ids, positions, block_tables, static_cast<unsigned char*>(kv_pool),
              out_next_ids, out_logits};
  if (use_stream(h, batch)) return run_stream(h, sp, h->stream);
  if (!h->cfg.use_graphs) return record_step(h, sp, nullptr, h->stream);

  GraphKey key{batch, {token_ids, positions, block_tables, kv_pool, out_next_ids, out_logits}};
  auto it = h->graphs.find(key);
  if (it == h->graphs.end()) {
    if (h->graphs.size() >= (size_t)kMaxGraphs) {
      // at the cap: destroy the least recently replayed graph (once the
      // stream has finished with it)
      auto old = h->graphs.begin();
      for (auto g = h->graphs.begin(); g != h->graphs.end(); ++g)
        if (h->graph_use[g->first] < h->graph_use[old->first]) old = g;
      HIP_TRY(h, hipStreamSynchronize(h->stream));
      (void)hipGraphExecDestroy(old->second);
      (void)hipGraphDestroy(h->graph_defs[old->first]);
      h->graph_defs.erase(old->first);
      h->graph_use.erase(old->first);
      h->graphs.erase(old);
    }
    // First call for this key: run it eagerly (this produces the results),
    // then capture the same launches on the private stream.
    if ((rc = record_step(h, sp, nullptr, h->stream))) return rc;
    HIP_TRY(h, hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal));
    rc = record_step(h, sp, nullptr, h->cap);
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(h->cap, &g);
    if (rc) { if (g) (void)hipGraphDestroy(g); return rc; }
    if (e != hipSuccess) return hip_fail(h, e, "hipStreamEndCapture");
    hipGraphExec_t ge = nullptr;
    e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
    if (e != hipSuccess) { (void)hipGraphDestroy(g); return hip_fail(h, e, "hipGraphInstantiate"); }
    h->graphs[key] = ge;
    h->graph_defs[key] = g;
    h->graph_use[key] = ++h->graph_clock;
    return QD_OK;
  }
  h->graph_use[key] = ++h->graph_clock;
  HIP_TRY(h, hipGraphLaunch(it->second, h->stream));
  return QD_OK;
}

int qd_prefill(qd_handle* h, int32_t rows, const int32_t* token_ids, const int32_t* positions,
               const int32_t* block_tables, void* kv_pool, int32_t n_logits,
               int32_t* out_next_ids, float* out_logits) {
  if (!h) return QD_EINVAL;
  if (n_logits < 0 || n_logits > rows) return fail(h, QD_EINVAL, "n_logits must be in 0..rows");
  if (n_logits > 0 && !out_next_ids) return fail(h, QD_EINVAL, "NULL out_next_ids");
  // (out_next_ids may be NULL here: token_ids stands in for it in the check)
  int rc = check_step_args(h, rows, token_ids, positions, block_tables, kv_pool, token_ids);
  if (rc) return rc;
  StepPtrs sp{rows, token_ids, positions, block_tables, static_cast<unsigned char*>(kv_pool),
              out_next_ids, out_logits, n_logits};
  return record_step(h, sp, nullptr, h->stream);
}

int qd_prefill_prompts(qd_handle* h, int32_t n_seqs, const int32_t* seq_rows,
                       const int32_t* start_pos, const int32_t* token_ids,
                       const int32_t* block_tables, void* kv_pool, int32_t n_logits,
                       int32_t* out_next_ids, float* out_logits) {
  if (!h) return QD_EINVAL;
  if (h->pf_rows == 0)
    return fail(h, QD_EUNSUPPORTED, "handle created with max_prefill_rows = 0");
  if (n_seqs < 1 || n_seqs > kPfMaxSegs) return fail(h, QD_EINVAL, "n_seqs must be in 1..64");
  if (!seq_rows || !start_pos || !token_ids || !block_tables || !kv_pool)
    return fail(h, QD_EINVAL, "NULL prefill pointer");
  if (n_logits < 0 || n_logits > n_seqs || n_logits > h->cfg.max_batch)
    return fail(h, QD_EINVAL, "n_logits must be in 0..min(n_seqs, max_batch)");
  if (n_logits > 0 && !out_next_ids) return fail(h, QD_EINVAL, "NULL out_next_ids");
  std::string missing;
  if (!all_loaded(h, &missing)) return fail(h, QD_ESTATE, "weight not loaded: " + missing);
  PfSegs sg{};
  sg.n = n_seqs;
  long long rows = 0, qb = 0;
  for (int s = 0; s < n_seqs; ++s) {
    if (seq_rows[s] < 1) return fail(h, QD_EINVAL, "seq_rows must be >= 1");
    if (start_pos[s] < 0 || (long long)start_pos[s] + seq_rows[s] > h->max_pos)
      return fail(h, QD_EINVAL, "segment positions past max_pages_per_seq * 16");
    sg.row0[s] = (int)rows;
    sg.pos0[s] = start_pos[s];
    sg.qb0[s] = (int)qb;
    rows += seq_rows[s];
    qb += (seq_rows[s] + 15) / 16;
    if (rows > h->cfg.max_prefill_rows)
      return fail(h, QD_EINVAL, "rows of all segments exceed max_prefill_rows");
  }
  sg.row0[n_seqs] = (int)rows;
  sg.qb0[n_seqs] = (int)qb;
  return record_prefill_prompts(h, sg, token_ids, block_tables, static_cast<unsigned char*>(kv_pool),
                                n_logits, out_next_ids, out_logits);
}

int qd_profile_step(qd_handle* h, int32_t batch, const int32_t* token_ids,
                    const int32_t* positions, const int32_t* block_tables, void* kv_pool,
                    int32_t* out_next_ids, float* out_logits, float* class_ms,
                    int32_t* class_launches) {
  int rc = check_step_args(h, batch, token_ids, positions, block_tables, kv_pool, out_next_ids);
  if (rc) return rc;
  if (!class_ms || !class_launches) return fail(h, QD_EINVAL, "NULL profile output");
  StepPtrs sp{batch, token_ids, positions, block_tables, static_cast<unsigned char*>(kv_pool),
              out_next_ids, out_logits};
  // The step is enqueued twice: while the GPU runs the first copy, the host
  // has time to enqueue the second, profiled one completely, so its kernels
  // run back to back without host launch gaps between the events.  (Events
  // recorded inside a captured graph cannot be timed.)  Running the step
  // twice has the effects of running it once: it rewrites the same KV slot
  // with the same values.
  Prof pr;
  rc = record_step(h, sp, nullptr, h->stream);
  if (rc == QD_OK) rc = record_step(h, sp, nullptr, h->stream, &pr);
  hipError_t e = hipStreamSynchronize(h->stream);
  for (int c = 0; c < QD_PROF_CLASSES; ++c) { class_ms[c] = 0.f; class_launches[c] = 0; }
  if (rc == QD_OK && e == hipSuccess) {
    for (size_t i = 1; i < pr.ev.size(); ++i) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, pr.ev[i - 1], pr.ev[i]);
      if (e != hipSuccess) break;
      const int c = pr.cls[i];
      if (c >= 0 && c < QD_PROF_CLASSES) { class_ms[c] += ms; class_launches[c] += 1; }
    }
  }
  for (hipEvent_t ev : pr.ev) (void)hipEventDestroy(ev);
  if (rc) return rc;
  if (e != hipSuccess) return hip_fail(h, e, "profile events");
  return QD_OK;
}

int qd_profile_class(qd_handle* h, int32_t batch, int32_t cls, int32_t reps, float* avg_us) {
  if (!h || !avg_us) return QD_EINVAL;
  if (batch < 1 || batch > h->cfg.max_batch) return fail(h, QD_EINVAL, "batch out of range");
  if (reps < 1) return fail(h, QD_EINVAL, "reps must be >= 1");
  if (cls != QD_PROF_QKV && cls != QD_PROF_O && cls != QD_PROF_GATE_UP && cls != QD_PROF_DOWN &&
      cls != QD_PROF_LM_HEAD)
    return fail(h, QD_EUNSUPPORTED, "only projection classes can be timed alone");
  std::string missing;
  if (!all_loaded(h, &missing)) return fail(h, QD_ESTATE, "weight not loaded: " + missing);
  const int n = cls == QD_PROF_LM_HEAD ? 1 : h->L;
  hipGraph_t g = nullptr;
  hipGraphExec_t ge = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = QD_OK;
  hipError_t e = hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(h, e, "hipStreamBeginCapture");
  for (int l = 0; l < n && e == hipSuccess; ++l)
    e = launch_projection(h, batch, cls, l, true, nullptr, h->prof_ids, h->cap);
  hipError_t e2 = hipStreamEndCapture(h->cap, &g);
  if (e == hipSuccess) e = e2;
  if (e == hipSuccess) e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = hipGraphLaunch(ge, h->stream);  // warm-up
  if (e == hipSuccess) e = hipEventRecord(e0, h->stream);
  for (int r = 0; r < reps && e == hipSuccess; ++r) e = hipGraphLaunch(ge, h->stream);
  if (e == hipSuccess) e = hipEventRecord(e1, h->stream);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e == hipSuccess) *avg_us = ms * 1e3f / (float)(reps * n);
  else rc = hip_fail(h, e, "qd_profile_class");
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (ge) (void)hipGraphExecDestroy(ge);
  if (g) (void)hipGraphDestroy(g);
  return rc;
}

int qd_sample(qd_handle* h, int32_t batch, const float* logits, const float* temperature,
              const int32_t* top_k, const float* top_p, const float* uniform,
              int32_t* out_ids) {
  if (!h) return QD_EINVAL;
  if (batch < 1 || batch > h->cfg.max_batch) return fail(h, QD_EINVAL, "batch out of range");
  if (!logits || !temperature || !top_k || !top_p || !uniform || !out_ids)
    return fail(h, QD_EINVAL, "NULL sampling pointer");
  if (reinterpret_cast<uintptr_t>(logits) % 16)
    return fail(h, QD_EINVAL, "logits must be 16-byte aligned");
  SampleArgs a{logits, h->V, temperature, top_k, top_p, uniform, out_ids,
               h->sample_G, h->sample_C, h->sample_max, h->sample_idx,
               h->sample_cand, h->sample_cnt, h->sample_sum, h->sample_cnt2,
               h->sample_hist, h->sample_pass_hist, h->sample_sum2, h->sample_sum3,
               h->sample_cnt3, h->sample_flag, h->sample_cut, h->dev_flags};
  HIP_TRY(h, launch_sample(a, batch, h->stream));
  return QD_OK;
}

int qd_read_ceiling(const void* buf, int64_t bytes, int32_t reps, void* hip_stream,
                    float* gbps) {
  if (!buf || !gbps || bytes < 1024 || reps < 1) return fail(nullptr, QD_EINVAL, "bad arguments");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  float best = 0.f;
  for (int per_cu = 1; per_cu <= 4 && e == hipSuccess; per_cu *= 2) {
    const int grid = per_cu * cus;
    e = launch_read_ceiling(buf, (size_t)bytes, grid, s);  // warm-up
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch_read_ceiling(buf, (size_t)bytes, grid, s);
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && ms > 0.f) {
      const float g = (float)((double)(bytes / 1024 * 1024) * reps / (ms * 1e-3) / 1e9);
      best = g > best ? g : best;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return hip_fail(nullptr, e, "qd_read_ceiling");
  *gbps = best;
  return QD_OK;
}

int qd_device_status(qd_handle* h, int32_t* flags) {
  if (!h || !flags) return QD_EINVAL;
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  int v = 0;
  HIP_TRY(h, hipMemcpy(&v, h->dev_flags, sizeof(int), hipMemcpyDeviceToHost));
  HIP_TRY(h, hipMemset(h->dev_flags, 0, sizeof(int)));
  *flags = v;
  return QD_OK;
}

void* qd_stream(const qd_handle* h) { return h ? static_cast<void*>(h->stream) : nullptr; }

int qd_step_path(const qd_handle* h, int32_t batch) {
  if (!h || batch < 1 || batch > h->cfg.max_batch) return QD_EINVAL;
  if (use_stream(h, batch)) return QD_PATH_STREAM;
  return h->cfg.use_graphs ? QD_PATH_GRAPH : QD_PATH_STAGED;
}

void qd_destroy(qd_handle* h) {
  if (!h) return;
  if (h->stream || h->cap) {
    (void)hipStreamSynchronize(h->stream);
  }
  for (auto& kv : h->graphs) (void)hipGraphExecDestroy(kv.second);
  for (auto& kv : h->graph_defs) (void)hipGraphDestroy(kv.second);
  for (void* p : h->allocs) (void)hipFree(p);
  if (h->cap) (void)hipStreamDestroy(h->cap);
  delete h;
}

const char* qd_last_error(const qd_handle* h) {
  return h ? h->err.c_str() : g_create_error.c_str();
}

}  // extern "C"
