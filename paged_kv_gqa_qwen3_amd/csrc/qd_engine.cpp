// Serving loop around the decode step: iteration-level (continuous)
// batching.  Requests wait in arrival order; each iteration admits as many
// as the batch has room for, prefills their prompts (a prefix found in the
// page cache is not prefilled again), runs one decode step for every
// request that already has a token, and hands the new tokens back.  A
// request joins the decode batch in the iteration after its prompt is done
// and leaves it on its end-of-sequence token or its token limit, so the
// batch size changes from one iteration to the next (the locsic page
// "推理引擎里面发生了什么", section Continuous Batching; the rkmt page
// "从零构建 Qwen3-8B 推理引擎", sections 4.3.2 on the batching scheduler and
// 4.4.4 on the automatic prefix cache).
//
// Host C++ over the public ABI of qd.h (qd_blocks_*, qd_prefill_prompts,
// qd_decode_step); every step of the model runs in the library's kernels.
// The engine's device buffers never move, so qd_decode_step replays one
// captured graph per batch size.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <string>
#include <unordered_map>
#include <vector>

#include "qd.h"
#include "qd_internal.h"

namespace {

constexpr int kPageTokens = 16;
constexpr int kMaxSegs = 64;  // prompt segments per qd_prefill_prompts call

enum class St { Waiting, Prefill, Decode };

struct Req {
  std::vector<int32_t> tokens;  // the prompt, then every token generated so far
  int32_t n_prompt = 0;
  int32_t max_new = 0;
  int32_t eos = -1;
  float temperature = 0.f;  // <= 0: greedy
  int32_t top_k = 0;
  float top_p = 1.f;
  uint64_t seed = 0;
  int32_t cached = 0;  // positions whose K/V are in the pool
  int32_t n_gen = 0;
  St st = St::Waiting;
};

struct Seg {
  int64_t id;
  int32_t start, rows;
  bool ends;
};

}  // namespace

struct qd_engine {
  qd_handle* h = nullptr;
  void* pool = nullptr;
  hipStream_t stream = nullptr;
  qd_blocks* blocks = nullptr;
  int max_batch = 0, mpps = 0, max_rows = 0, vocab = 0, num_pages = 0;
  bool broken = false;

  std::deque<int64_t> waiting;
  std::vector<int64_t> active;  // admitted, in admission order
  std::unordered_map<int64_t, Req> reqs;
  qd_engine_stats stats{};

  // decode inputs [tokens max_batch][positions max_batch][tables max_batch*mpps],
  // prompt inputs [tables kMaxSegs*mpps][tokens max_rows], the next ids
  // [prompt-ending segments kMaxSegs][decode rows max_batch], and the
  // sampling rows [temperature | top_k | top_p | uniform | sampled id], 2 *
  // max_batch each; each in device memory and in a pinned host mirror
  int32_t *d_dec = nullptr, *h_dec = nullptr;
  int32_t *d_pf = nullptr, *h_pf = nullptr;
  int32_t *d_out = nullptr, *h_out = nullptr;
  int32_t *d_sp = nullptr, *h_sp = nullptr;
  // logits of an iteration that samples: [2 * max_batch][vocab]; the decode
  // rows always at rows max_batch.., the n prompt-ending rows just before
  // them, so that one qd_sample call covers both
  float* d_logits = nullptr;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;  // an iteration's GPU span
  double gpu_us = 0.0;

  // host scratch reused by every iteration
  std::vector<Seg> segs;
  std::vector<int64_t> dec_ids, seg_ids;
  std::vector<int32_t> seg_rows, seg_start;
};

namespace {

int efail(qd_engine* e, int code, const std::string& msg) {
  return qd::handle_fail(e->h, code, "qd_engine: " + msg);
}

int ehip(qd_engine* e, hipError_t err, const char* what) {
  e->broken = true;
  return efail(e, QD_EHIP, std::string(what) + ": " + hipGetErrorString(err));
}

#define ENG_HIP(e, expr)                              \
  do {                                                \
    hipError_t err_ = (expr);                         \
    if (err_ != hipSuccess) return ehip((e), err_, #expr); \
  } while (0)

void free_buffers(qd_engine* e) {
  for (int32_t* p : {e->d_dec, e->d_pf, e->d_out, e->d_sp})
    if (p) (void)hipFree(p);
  for (int32_t* p : {e->h_dec, e->h_pf, e->h_out, e->h_sp})
    if (p) (void)hipHostFree(p);
  if (e->d_logits) (void)hipFree(e->d_logits);
  if (e->ev0) (void)hipEventDestroy(e->ev0);
  if (e->ev1) (void)hipEventDestroy(e->ev1);
  e->ev0 = e->ev1 = nullptr;
  e->d_dec = e->d_pf = e->d_out = e->d_sp = nullptr;
  e->h_dec = e->h_pf = e->h_out = e->h_sp = nullptr;
  e->d_logits = nullptr;
}

// The uniform draw for a request's k-th generated token: SplitMix64 (the
// splittable generator of Steele, Lea and Flood, as Vigna's 64-bit mixer)
// at state seed + (k + 1) * 0x9E3779B97F4A7C15, its top 24 bits as a float
// in [0, 1).
float draw(uint64_t seed, int32_t k) {
  uint64_t z = seed + (uint64_t)(k + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (float)(z >> 40) * (1.0f / 16777216.0f);
}

size_t dec_words(const qd_engine* e) { return (size_t)e->max_batch * (2 + e->mpps); }
size_t pf_words(const qd_engine* e) { return (size_t)kMaxSegs * e->mpps + e->max_rows; }
size_t out_words(const qd_engine* e) { return (size_t)kMaxSegs + e->max_batch; }
size_t sp_words(const qd_engine* e) { return (size_t)5 * 2 * e->max_batch; }

// A request leaves: its pages become cache entries for the tokens whose K/V
// they hold (the prompt and every generated token but the last, which was
// never decoded), then return to the pool.
int retire(qd_engine* e, int64_t id) {
  Req& r = e->reqs[id];
  int rc = qd_blocks_publish(e->blocks, id, r.tokens.data(), r.cached);
  if (rc >= 0) rc = qd_blocks_release(e->blocks, id);
  if (rc < 0) {
    e->broken = true;
    return efail(e, rc, "page manager refused to retire a request");
  }
  e->reqs.erase(id);
  e->active.erase(std::find(e->active.begin(), e->active.end(), id));
  return QD_OK;
}

// Admit waiting requests in arrival order while the batch has room.  A
// request takes every page it can need up front (prompt plus token limit),
// so a running request never waits for a page and nothing is preempted;
// when the pool cannot supply them it stays first in line until requests
// leave.  The prefix cache may supply the first full pages of the prompt,
// never its last token, whose logits start decoding.
int admit(qd_engine* e) {
  while (!e->waiting.empty() && (int)e->active.size() < e->max_batch) {
    const int64_t id = e->waiting.front();
    Req& r = e->reqs[id];
    int rc = qd_blocks_add(e->blocks, id);
    if (rc == QD_OK) rc = qd_blocks_match(e->blocks, id, r.tokens.data(), r.n_prompt - 1);
    if (rc < 0) {
      e->broken = true;
      return efail(e, rc, "page manager refused a new request");
    }
    const int32_t hit = rc;
    rc = qd_blocks_reserve(e->blocks, id, r.n_prompt + r.max_new - 1);
    if (rc == QD_ENOMEM) {
      if (qd_blocks_release(e->blocks, id) < 0) {
        e->broken = true;
        return efail(e, QD_EINVAL, "page manager refused a release");
      }
      break;
    }
    if (rc < 0) {
      e->broken = true;
      return efail(e, rc, "page manager refused a reservation");
    }
    r.cached = hit;
    r.st = St::Prefill;
    e->stats.cached_rows += hit;
    e->active.push_back(id);
    e->waiting.pop_front();
  }
  return QD_OK;
}

}  // namespace

extern "C" {

int qd_engine_create(qd_handle* h, void* kv_pool, qd_engine** out) {
  if (!h || !kv_pool || !out) return h ? qd::handle_fail(h, QD_EINVAL, "qd_engine: NULL argument")
                                       : QD_EINVAL;
  *out = nullptr;
  const qd_config* c = qd::handle_config(h);
  if (c->max_prefill_rows < 1)
    return qd::handle_fail(h, QD_EUNSUPPORTED,
                           "qd_engine: the handle needs max_prefill_rows >= 1 for prompts");
  qd_engine* e = new qd_engine;
  e->h = h;
  e->pool = kv_pool;
  e->stream = static_cast<hipStream_t>(qd_stream(h));
  e->max_batch = c->max_batch;
  e->mpps = c->max_pages_per_seq;
  e->max_rows = c->max_prefill_rows;
  e->vocab = c->vocab;
  e->num_pages = c->num_pages;
  int rc = qd_blocks_create(c->num_pages, c->max_pages_per_seq, &e->blocks);
  if (rc != QD_OK) {
    delete e;
    return qd::handle_fail(h, rc, "qd_engine: page manager");
  }
  hipError_t err = hipSuccess;
  const size_t bytes[4] = {dec_words(e) * 4, pf_words(e) * 4, out_words(e) * 4, sp_words(e) * 4};
  int32_t** dev[4] = {&e->d_dec, &e->d_pf, &e->d_out, &e->d_sp};
  int32_t** host[4] = {&e->h_dec, &e->h_pf, &e->h_out, &e->h_sp};
  if (err == hipSuccess)
    err = hipMalloc(reinterpret_cast<void**>(&e->d_logits), (size_t)2 * e->max_batch * e->vocab * 4);
  if (err == hipSuccess) err = hipEventCreate(&e->ev0);
  if (err == hipSuccess) err = hipEventCreate(&e->ev1);
  for (int i = 0; i < 4 && err == hipSuccess; ++i) {
    err = hipMalloc(reinterpret_cast<void**>(dev[i]), bytes[i]);
    if (err == hipSuccess) err = hipHostMalloc(reinterpret_cast<void**>(host[i]), bytes[i], 0);
    if (err == hipSuccess) std::memset(*host[i], 0, bytes[i]);
    if (err == hipSuccess) err = hipMemset(*dev[i], 0, bytes[i]);
  }
  if (err != hipSuccess) {
    free_buffers(e);
    qd_blocks_destroy(e->blocks);
    delete e;
    return qd::handle_fail(h, err == hipErrorOutOfMemory ? QD_ENOMEM : QD_EHIP,
                           std::string("qd_engine: buffers: ") + hipGetErrorString(err));
  }
  e->segs.reserve(kMaxSegs);
  *out = e;
  return QD_OK;
}

void qd_engine_destroy(qd_engine* e) {
  if (!e) return;
  if (e->stream) (void)hipStreamSynchronize(e->stream);
  free_buffers(e);
  qd_blocks_destroy(e->blocks);
  delete e;
}

int qd_engine_submit(qd_engine* e, const qd_engine_request* rq) {
  if (!e) return QD_EINVAL;
  if (e->broken) return efail(e, QD_ESTATE, "an earlier failure left the engine unusable");
  if (!rq) return efail(e, QD_EINVAL, "NULL request");
  const int32_t n_prompt = rq->n_prompt, max_new_tokens = rq->max_new_tokens;
  const int32_t* prompt = rq->prompt;
  if (!prompt || n_prompt < 1) return efail(e, QD_EINVAL, "empty or NULL prompt");
  if (max_new_tokens < 1) return efail(e, QD_EINVAL, "max_new_tokens must be >= 1");
  if (rq->eos_id < -1 || rq->eos_id >= e->vocab)
    return efail(e, QD_EINVAL, "eos_id outside -1..vocab-1");
  if (e->reqs.count(rq->id)) return efail(e, QD_EINVAL, "request id already in use");
  const int64_t span = (int64_t)n_prompt + max_new_tokens - 1;
  if (span > (int64_t)e->mpps * kPageTokens)
    return efail(e, QD_EUNSUPPORTED, "prompt plus max_new_tokens exceed max_pages_per_seq * 16");
  if ((span + kPageTokens - 1) / kPageTokens > e->num_pages)
    return efail(e, QD_EUNSUPPORTED, "prompt plus max_new_tokens need more pages than the pool has");
  for (int32_t i = 0; i < n_prompt; ++i)
    if (prompt[i] < 0 || prompt[i] >= e->vocab) return efail(e, QD_EINVAL, "prompt token outside the vocabulary");
  Req r;
  r.tokens.assign(prompt, prompt + n_prompt);
  r.tokens.reserve((size_t)n_prompt + max_new_tokens);
  r.n_prompt = n_prompt;
  r.max_new = max_new_tokens;
  r.eos = rq->eos_id;
  r.temperature = rq->temperature;
  r.top_k = rq->top_k;
  r.top_p = rq->top_p;
  r.seed = rq->seed;
  e->reqs.emplace(rq->id, std::move(r));
  e->waiting.push_back(rq->id);
  return QD_OK;
}

int qd_engine_step(qd_engine* e, int32_t max_out, int64_t* out_req, int32_t* out_token,
                   int32_t* out_done, int32_t* n_out) {
  if (!e) return QD_EINVAL;
  if (e->broken) return efail(e, QD_ESTATE, "an earlier failure left the engine unusable");
  if (!out_req || !out_token || !out_done || !n_out) return efail(e, QD_EINVAL, "NULL output");
  if (max_out < e->max_batch) return efail(e, QD_EINVAL, "max_out must be >= max_batch");
  *n_out = 0;
  int rc = admit(e);
  if (rc) return rc;
  if (e->active.empty()) return QD_OK;

  // Prompt rows of this iteration: requests still prefilling, in admission
  // order, each as much of its remaining prompt as the row budget allows
  // (a long prompt continues over several iterations).  Segments that end
  // a prompt go first: their last rows get logits.
  e->segs.clear();
  e->dec_ids.clear();
  int32_t budget = e->max_rows;
  for (int64_t id : e->active) {
    Req& r = e->reqs[id];
    if (r.st == St::Decode) {
      e->dec_ids.push_back(id);
    } else if (budget > 0 && (int)e->segs.size() < kMaxSegs) {
      const int32_t rem = r.n_prompt - r.cached;
      const int32_t rows = std::min(rem, budget);
      e->segs.push_back({id, r.cached, rows, rows == rem});
      budget -= rows;
    }
  }
  std::stable_partition(e->segs.begin(), e->segs.end(), [](const Seg& s) { return s.ends; });
  const int n_seg = (int)e->segs.size();
  const int n_end = (int)std::count_if(e->segs.begin(), e->segs.end(), [](const Seg& s) { return s.ends; });
  const int B = (int)e->dec_ids.size();

  // An iteration samples when one of the requests that gets a token here
  // does (temperature > 0): the steps then also write logits, prompt rows
  // just before the decode rows, for one qd_sample call over all of them.
  bool sample = false;
  for (int s = 0; s < n_end; ++s) sample |= e->reqs[e->segs[s].id].temperature > 0.f;
  for (int b = 0; b < B; ++b) sample |= e->reqs[e->dec_ids[b]].temperature > 0.f;
  const int mb = e->max_batch, r0 = mb - n_end;  // first sampled row
  float* const lg_pf = sample && n_end > 0 ? e->d_logits + (size_t)r0 * e->vocab : nullptr;
  float* const lg_dec = sample ? e->d_logits + (size_t)mb * e->vocab : nullptr;

  const size_t tab = (size_t)kMaxSegs * e->mpps;
  ENG_HIP(e, hipEventRecord(e->ev0, e->stream));
  if (n_seg > 0) {
    e->seg_ids.clear();
    e->seg_rows.clear();
    e->seg_start.clear();
    int32_t* tok = e->h_pf + tab;
    int32_t row = 0;
    for (const Seg& s : e->segs) {
      e->seg_ids.push_back(s.id);
      e->seg_rows.push_back(s.rows);
      e->seg_start.push_back(s.start);
      std::memcpy(tok + row, e->reqs[s.id].tokens.data() + s.start, (size_t)s.rows * 4);
      row += s.rows;
    }
    rc = qd_blocks_tables(e->blocks, e->seg_ids.data(), n_seg, 0, e->h_pf);
    if (rc < 0) {
      e->broken = true;
      return efail(e, rc, "page manager refused the prompt tables");
    }
    ENG_HIP(e, hipMemcpyAsync(e->d_pf, e->h_pf, (size_t)n_seg * e->mpps * 4, hipMemcpyHostToDevice,
                              e->stream));
    ENG_HIP(e, hipMemcpyAsync(e->d_pf + tab, tok, (size_t)row * 4, hipMemcpyHostToDevice, e->stream));
    rc = qd_prefill_prompts(e->h, n_seg, e->seg_rows.data(), e->seg_start.data(), e->d_pf + tab,
                            e->d_pf, e->pool, n_end, n_end ? e->d_out : nullptr, lg_pf);
    if (rc) {
      e->broken = true;
      return rc;
    }
    e->stats.prefill_rows += row;
  }
  if (B > 0) {
    int32_t* tok = e->h_dec;
    int32_t* pos = e->h_dec + e->max_batch;
    for (int b = 0; b < B; ++b) {
      const Req& r = e->reqs[e->dec_ids[b]];
      tok[b] = r.tokens.back();
      pos[b] = r.cached;
    }
    rc = qd_blocks_tables(e->blocks, e->dec_ids.data(), B, 0, e->h_dec + 2 * e->max_batch);
    if (rc < 0) {
      e->broken = true;
      return efail(e, rc, "page manager refused the decode tables");
    }
    ENG_HIP(e, hipMemcpyAsync(e->d_dec, e->h_dec, ((size_t)2 * e->max_batch + (size_t)B * e->mpps) * 4,
                              hipMemcpyHostToDevice, e->stream));
    rc = qd_decode_step(e->h, B, e->d_dec, e->d_dec + e->max_batch, e->d_dec + 2 * e->max_batch, e->pool,
                        e->d_out + kMaxSegs, lg_dec);
    if (rc) {
      e->broken = true;
      return rc;
    }
    e->stats.decode_rows += B;
  }
  // sampling rows [temperature | top_k | top_p | uniform | id], 2 * max_batch each
  const int R2 = 2 * mb;
  float* const sp_t = reinterpret_cast<float*>(e->h_sp);
  int32_t* const sp_k = e->h_sp + R2;
  float* const sp_p = reinterpret_cast<float*>(e->h_sp + 2 * R2);
  float* const sp_u = reinterpret_cast<float*>(e->h_sp + 3 * R2);
  int32_t* const sp_id = e->h_sp + 4 * R2;
  if (sample) {
    auto row = [&](int r, const Req& q) {
      sp_t[r] = q.temperature;
      sp_k[r] = q.top_k;
      sp_p[r] = q.top_p;
      sp_u[r] = draw(q.seed, q.n_gen);
    };
    for (int s = 0; s < n_end; ++s) row(r0 + s, e->reqs[e->segs[s].id]);
    for (int b = 0; b < B; ++b) row(mb + b, e->reqs[e->dec_ids[b]]);
    ENG_HIP(e, hipMemcpyAsync(e->d_sp, e->h_sp, (size_t)4 * R2 * 4, hipMemcpyHostToDevice, e->stream));
    const int32_t* d_sp = e->d_sp;
    rc = qd_sample(e->h, n_end + B, e->d_logits + (size_t)r0 * e->vocab,
                   reinterpret_cast<const float*>(d_sp) + r0, d_sp + R2 + r0,
                   reinterpret_cast<const float*>(d_sp + 2 * R2) + r0,
                   reinterpret_cast<const float*>(d_sp + 3 * R2) + r0, e->d_sp + 4 * R2 + r0);
    if (rc) {
      e->broken = true;
      return rc;
    }
    ENG_HIP(e, hipEventRecord(e->ev1, e->stream));
    ENG_HIP(e, hipMemcpyAsync(sp_id + r0, e->d_sp + 4 * R2 + r0, (size_t)(n_end + B) * 4,
                              hipMemcpyDeviceToHost, e->stream));
  } else {
    ENG_HIP(e, hipEventRecord(e->ev1, e->stream));
    if (n_end > 0)
      ENG_HIP(e, hipMemcpyAsync(e->h_out, e->d_out, (size_t)n_end * 4, hipMemcpyDeviceToHost, e->stream));
    if (B > 0)
      ENG_HIP(e, hipMemcpyAsync(e->h_out + kMaxSegs, e->d_out + kMaxSegs, (size_t)B * 4,
                                hipMemcpyDeviceToHost, e->stream));
  }
  int32_t flags = 0;
  rc = qd_device_status(e->h, &flags);  // waits for the stream
  if (rc) {
    e->broken = true;
    return rc;
  }
  if (flags) {
    e->broken = true;
    return efail(e, QD_EHIP, "the kernels reported device status flags " + std::to_string(flags));
  }
  e->stats.steps += 1;
  {
    float ms = 0.f;
    ENG_HIP(e, hipEventElapsedTime(&ms, e->ev0, e->ev1));
    e->gpu_us += 1e3 * ms;
  }

  // Hand out the tokens: decode rows first, then the first token of every
  // prompt that ended; a request that reached its limit or its
  // end-of-sequence token leaves.
  int n = 0;
  std::vector<int64_t>& done = e->seg_ids;  // reused: ids that leave this iteration
  done.clear();
  auto emit = [&](int64_t id, Req& r, int32_t t) {
    r.tokens.push_back(t);
    r.n_gen += 1;
    const bool fin = r.n_gen >= r.max_new || t == r.eos;
    out_req[n] = id;
    out_token[n] = t;
    out_done[n] = fin ? 1 : 0;
    ++n;
    if (fin) done.push_back(id);
  };
  for (int b = 0; b < B; ++b) {
    Req& r = e->reqs[e->dec_ids[b]];
    r.cached += 1;
    emit(e->dec_ids[b], r, sample ? sp_id[mb + b] : e->h_out[kMaxSegs + b]);
  }
  for (int s = 0; s < n_seg; ++s) {
    const Seg& sg = e->segs[s];
    Req& r = e->reqs[sg.id];
    r.cached = sg.start + sg.rows;
    if (sg.ends) {
      r.st = St::Decode;
      emit(sg.id, r, sample ? sp_id[r0 + s] : e->h_out[s]);
    }
  }
  e->stats.tokens_out += n;
  if (sample) e->stats.sampled_iterations += 1;
  for (int64_t id : done) {
    rc = retire(e, id);
    if (rc) return rc;
  }
  *n_out = n;
  return QD_OK;
}

int qd_engine_get_stats(const qd_engine* e, qd_engine_stats* out) {
  if (!e || !out) return QD_EINVAL;
  *out = e->stats;
  out->gpu_us = (int64_t)e->gpu_us;
  out->waiting = (int32_t)e->waiting.size();
  out->running = (int32_t)e->active.size();
  out->pages_available = qd_blocks_available(e->blocks);
  return QD_OK;
}

}  // extern "C"
