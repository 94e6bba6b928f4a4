// On-device sampling of the next token from one row of logits per
// workgroup: temperature, top-k and top-p, with a uniform draw the caller
// supplies, so that only the token id leaves the GPU (the yuzheng310 page,
// "GPU 算子与执行优化", part 3: argmax and the top-p/top-k filters stay on
// the device; the rkmt page, section 4.1.2: temperature and top_p travel with
// a request, the sampled token comes back).
//
// The pages fix no algorithm; the kernel follows the plain definitions:
//   * temperature <= 0 (or NaN): the greedy token, lowest index on ties;
//   * weights w_i = exp((l_i - max l) / T) in fp32, held as integers
//     q_i = floor(w_i * 2^32) (kept in doubles: every sum stays below 2^53,
//     so sums are exact and independent of order);
//   * rank order: logit descending, then token id ascending;
//   * top_k in 1..V-1 keeps the first top_k tokens in rank order;
//   * top_p < 1 keeps, of those, the shortest rank-order prefix whose weight
//     reaches ceil(top_p * Q) (Q: the weight top-k kept; top_p <= 0: the
//     first token alone);
//   * the draw: t = min(floor(u * R), R - 1) over the kept weight R, and the
//     token is the kept one, in increasing id order, whose running weight
//     first exceeds t.
//
// Three launches per call, G workgroups per row (G = ceil(V / 8192)), each
// owning a chunk of at most 8192 logits.
//   First launch: every chunk loads its logits into LDS once and leaves its
//   (max, argmax) and, for 2 <= top_k <= kFastTopK or for top-p without
//   top_k, its 64 first tokens in rank order (each wave sorts batches of 64
//   across its lanes and keeps the best 64; the waves' lists are merged).
//   The last workgroup of the row to arrive takes the greedy token from the
//   maxima, or, with 2 <= top_k <= kFastTopK, merges the chunks' lists into
//   the row's first 64 tokens and takes top-k, top-p and the draw in one
//   wave.
//   Second launch, rows without top_k: every chunk sums its weights against
//   the row's max (with top-p also its weight per top key byte, added into
//   the row's histogram); the last workgroup then walks the chunk holding
//   the draw target (no limit), or takes the top-p cut and the draw over
//   the row's first 64 tokens when they reach the target.
//   Third launch, the rest: top-p rows whose nucleus goes beyond the first
//   64 tokens, and top_k above kFastTopK.  All G workgroups of the row take
//   the cut points in rank order by radix selection over a 32-bit key that
//   orders floats (four passes of 8 bits: token counts for top-k, then
//   weight for top-p; for top-p alone the first pass is the second launch's
//   histogram), then each cut id and the draw in id order, each chunk from
//   LDS, with barriers between the steps.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "qd_device.h"

namespace qd {

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / 64;

// Larger float -> larger key; -0 and +0 share a key (they rank as equals).
__device__ __forceinline__ unsigned sample_key(float x) {
  const unsigned b = __float_as_uint(x + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct SampleSmem {
  double mass[256];
  double wd[kSampleWaves];
  float wv[kSampleWaves];
  int wi[kSampleWaves];
  unsigned key;       // a selected cut key
  double need;        // count or weight still to take at that key
  int id;             // last id kept at the cut key
};

__device__ __forceinline__ float key_value(unsigned key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Add val to histogram bin `bin` of sm.mass for the lanes where `on` (call
// in wave-uniform control flow): lanes of one bin are summed first while at
// least 8 share it (the top byte of the key puts most tokens of a row in a
// few bins), the rest add one by one.
__device__ __forceinline__ void hist_add(SampleSmem& sm, unsigned bin, double val, bool on) {
  const int lane = threadIdx.x & 63;
  unsigned long long pending = __ballot(on);
  while (pending) {
    const int leader = __ffsll((long long)pending) - 1;
    const unsigned lb = __shfl(bin, leader);
    const bool same = ((pending >> lane) & 1ull) && bin == lb;
    const unsigned long long m = __ballot(same);
    if (__popcll(m) < 8) {
      if ((pending >> lane) & 1ull) atomicAdd(&sm.mass[bin], val);
      break;
    }
    double sum = same ? val : 0.0;
#pragma unroll
    for (int s2 = 32; s2 >= 1; s2 >>= 1) sum += __shfl_xor(sum, s2);
    if (lane == leader) atomicAdd(&sm.mass[lb], sum);
    pending &= ~m;
  }
}

// After a histogram pass of a radix selection: the bin (from the top) whose
// running total reaches `need`, into sm.key (with the digits fixed so far)
// and what remains to take inside it into sm.need.  Threads 0-63 only.
__device__ __forceinline__ void pick_bin(SampleSmem& sm, unsigned prefix, int shift, double need) {
  const int lane = threadIdx.x & 63;
  double m4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) m4[e] = sm.mass[255 - (4 * lane + e)];
  const double s4 = m4[0] + m4[1] + m4[2] + m4[3];
  double inc = s4;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  double before = inc - s4;
  const unsigned long long hit = __ballot(before < need && need <= inc);
  const int first = hit ? __ffsll((long long)hit) - 1 : 63;
  if (lane == first) {
    int e = 0;
    while (e < 3 && before + m4[e] < need) { before += m4[e]; ++e; }
    const unsigned bin = 255u - (unsigned)(4 * lane + e);
    sm.key = prefix | (bin << shift);
    sm.need = need - before;
  }
}

// Sum over the block (exact: the values are integers below 2^53).
__device__ __forceinline__ double block_sum(double v, SampleSmem& sm) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) sm.wd[wave] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kSampleWaves; ++w) s += sm.wd[w];
  return s;
}

// Exclusive prefix over threads in thread order (exact, as block_sum).
__device__ __forceinline__ double block_exclusive(double v, SampleSmem& sm) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  __syncthreads();
  if (lane == 63) sm.wd[wave] = inc;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave; ++w) base += sm.wd[w];
  return base + inc - v;
}

// Top-64 lists, one value per lane, sorted descending across the lanes of a
// wave.  A token is the 64-bit value key << 32 | (2^32 - 1 - id): larger
// for a larger logit, then a lower id (the rank order); 0 is "no token".
typedef unsigned long long u64;
static_assert(kFastTopK <= 64, "the fast path keeps 64 candidates per chunk");
constexpr int kSurvivors = 1024;  // tokens of a chunk the fast path gathers past its bound

__device__ __forceinline__ u64 shfl64(u64 v, int src) {
  const unsigned lo = __shfl((unsigned)v, src), hi = __shfl((unsigned)(v >> 32), src);
  return ((u64)hi << 32) | lo;
}
__device__ __forceinline__ u64 shfl_xor64(u64 v, int m) {
  const unsigned lo = __shfl_xor((unsigned)v, m), hi = __shfl_xor((unsigned)(v >> 32), m);
  return ((u64)hi << 32) | lo;
}

// Bitonic sort of the wave's 64 values, descending across lanes.
__device__ __forceinline__ u64 sort64(u64 x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const u64 y = shfl_xor64(x, stride);
      const bool keep_max = ((lane & stride) == 0) == ((lane & size) == 0);
      x = keep_max ? (x > y ? x : y) : (x < y ? x : y);
    }
  return x;
}

// The 64 largest of two sorted lists, sorted: the lane-wise larger of one
// list and the other reversed is bitonic and holds them; a bitonic merge
// orders it.
__device__ __forceinline__ u64 merge64(u64 a, u64 b) {
  const int lane = threadIdx.x & 63;
  const u64 br = shfl64(b, 63 - lane);
  u64 x = a > br ? a : br;
#pragma unroll
  for (int stride = 32; stride > 0; stride >>= 1) {
    const u64 y = shfl_xor64(x, stride);
    x = (lane & stride) == 0 ? (x > y ? x : y) : (x < y ? x : y);
  }
  return x;
}

// Merge cnt sorted lists of 64 (list j at L + 64 * j, in LDS) into the
// first, pairwise in rounds, the waves of the workgroup taking the pairs of
// a round in parallel.  Every thread of the workgroup must call it.
__device__ __forceinline__ void merge_lists(u64* L, int cnt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int step = 1; step < cnt; step <<= 1) {
    for (int j = wave * 2 * step; j + step < cnt; j += kSampleWaves * 2 * step)
      L[64 * j + lane] = merge64(L[64 * j + lane], L[64 * (j + step) + lane]);
    __syncthreads();
  }
}

__device__ __forceinline__ u64 token_value(float l, int id) {
  return ((u64)sample_key(l) << 32) | (0xffffffffu - (unsigned)id);
}

__global__ __launch_bounds__(kSampleThreads) void sample_kernel(SampleArgs a) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ SampleSmem sm;
  __shared__ u64 lists[kSampleWaves][64];
  __shared__ u64 surv[kSurvivors];
  __shared__ u64 s_bound;
  __shared__ unsigned s_nsurv;
  __shared__ unsigned s_flag;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.G, b = blockIdx.x / G, g = blockIdx.x % G;
  const int V = a.V;
  const float T = a.temperature[b];
  const int k = a.top_k[b];
  const float p = a.top_p[b];
  float u = a.uniform[b];
  if (!(u >= 0.f)) u = 0.f;  // negative or NaN draws count as 0
  const bool greedy = !(T > 0.f) || p <= 0.f || k == 1;
  const bool fast = !greedy && k > 1 && k <= kFastTopK;
  // rows the second launch finishes: no limit, or top-p alone
  const bool plain = !greedy && (k <= 0 || k >= V) && !(p < 1.f);
  const bool topp = !greedy && (k <= 0 || k >= V) && p < 1.f;

  // --- this workgroup's chunk of the row into LDS (n is a multiple of 4)
  float* const xs = reinterpret_cast<float*>(dyn);
  const int c0 = g * a.C, n = max(0, min(a.C, V - c0));
  const f32x4* src = reinterpret_cast<const f32x4*>(a.logits + (size_t)b * V + c0);
  for (int j = tid; j < n / 4; j += kSampleThreads) reinterpret_cast<f32x4*>(xs)[j] = src[j];
  __syncthreads();

  // --- the chunk's max (lowest index on ties)
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = tid; i < n; i += kSampleThreads) amax_merge(bv, bi, xs[i], c0 + i);
  wave_amax(bv, bi);
  if (lane == 0) { sm.wv[wave] = bv; sm.wi[wave] = bi; }
  __syncthreads();
  for (int w = 0; w < kSampleWaves; ++w) amax_merge(bv, bi, sm.wv[w], sm.wi[w]);
  const size_t slot = (size_t)b * G + g;
  if (tid == 0) { st_agent(a.part_max + slot, bv); st_agent(a.part_idx + slot, bi); }

  // --- the chunk's 64 first tokens in rank order.  A bound first: thread
  // t's tokens are t, t + 1024, ...; the tokens of one lane index across the
  // waves form 64 disjoint groups, and the least of the 64 group maxima is
  // at most the chunk's 64th largest, so only tokens at or above it can be
  // among the first 64.  Those (a few hundred in practice) are gathered and
  // every wave sorts batches of 64 of them across its lanes, keeping the
  // best 64; the waves' lists are then merged.  If more than kSurvivors pass
  // the bound, every token of the chunk goes through the sorts instead.
  if (fast || topp) {
    u64 gm = 0ull;
    for (int i = tid; i < n; i += kSampleThreads) {
      const u64 v = token_value(xs[i], c0 + i);
      gm = v > gm ? v : gm;
    }
    lists[wave][lane] = gm;
    if (tid == 0) s_nsurv = 0u;
    __syncthreads();
    if (wave == 0) {
      for (int w = 1; w < kSampleWaves; ++w) gm = lists[w][lane] > gm ? lists[w][lane] : gm;
      u64 lo = gm;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const u64 o = shfl_xor64(lo, m);
        lo = o < lo ? o : lo;
      }
      if (lane == 0) s_bound = lo;
    }
    __syncthreads();
    const u64 bound = s_bound;
    for (int i = tid; i < n; i += kSampleThreads) {
      const u64 v = token_value(xs[i], c0 + i);
      if (v >= bound) {
        const unsigned at = atomicAdd(&s_nsurv, 1u);
        if (at < (unsigned)kSurvivors) surv[at] = v;
      }
    }
    __syncthreads();
    const int ns = (int)s_nsurv;
    u64 best = 0ull;
    if (ns <= kSurvivors) {
      for (int s0 = wave * 64; s0 < ns; s0 += kSampleWaves * 64) {
        const int i = s0 + lane;
        best = merge64(best, sort64(i < ns ? surv[i] : 0ull));
      }
    } else {
      const int per = (n + kSampleWaves - 1) / kSampleWaves;
      const int w_lo = min(n, wave * per), w_hi = min(n, w_lo + per);
      for (int s0 = w_lo; s0 < w_hi; s0 += 64) {
        const int i = s0 + lane;
        best = merge64(best, sort64(i < w_hi ? token_value(xs[i], c0 + i) : 0ull));
      }
    }
    __syncthreads();  // every wave is done with the group maxima in lists
    lists[wave][lane] = best;
    __syncthreads();
    merge_lists(&lists[0][0], kSampleWaves);
    if (wave == 0)
      __hip_atomic_store(a.cand + slot * 64 + lane, lists[0][lane], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  // --- the last workgroup of the row to arrive finishes it
  unsigned* const cnt = a.counters + (size_t)b * kCntStride;
  if (!arrive_last(cnt, (unsigned)G, &s_flag)) return;
  if (tid == 0) reset_counter(cnt);
  bv = -INFINITY;
  bi = 0x7fffffff;
  for (int w = tid; w < G; w += kSampleThreads)
    amax_merge(bv, bi, ld_agent(a.part_max + (size_t)b * G + w), ld_agent(a.part_idx + (size_t)b * G + w));
  wave_amax(bv, bi);
  __syncthreads();
  if (lane == 0) { sm.wv[wave] = bv; sm.wi[wave] = bi; }
  __syncthreads();
  for (int w = 0; w < kSampleWaves; ++w) amax_merge(bv, bi, sm.wv[w], sm.wi[w]);
  if (tid == 0) a.out[b] = bi;  // greedy, and the fallback of the draws below
  if (greedy) return;
  if (plain || topp) return;  // finished by the second launch
  if (!fast) return;  // top-k above kFastTopK: the third launch

  // Fast path: the chunks' lists into LDS (all loads in flight at once; the
  // chunk is no longer needed: G * 512 bytes <= 4 * C), merged pairwise by
  // all waves into the row's 64 first tokens in rank order; then wave 0,
  // lane r holding rank r, takes the weights of the first k, the top-p cut
  // in rank order and the draw in id order.
  const u64* lst = a.cand + (size_t)b * G * 64;
  u64* const cl = reinterpret_cast<u64*>(dyn);
  __syncthreads();  // every thread is done with the chunk
  for (int i = tid; i < G * 64; i += kSampleThreads)
    cl[i] = __hip_atomic_load(lst + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  merge_lists(cl, G);
  if (wave != 0) return;
  const u64 c = cl[lane];
  const bool in = lane < k && c != 0ull;
  const int id = (int)(0xffffffffu - (unsigned)c);
  const float l = key_value((unsigned)(c >> 32));
  const double w = in ? floor((double)expf((l - bv) / T) * 4294967296.0) : 0.0;
  double incl = w;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  const double Q = __shfl(incl, 63);
  int nkeep = k;
  if (p < 1.f) {
    const double target = ceil((double)p * Q);
    const unsigned long long hit = __ballot(in && incl >= target);
    if (hit) nkeep = __ffsll((long long)hit);
  }
  const double wk = lane < nkeep ? w : 0.0;
  double R = wk;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) R += __shfl_xor(R, m);
  const double t = fmin(floor((double)u * R), R - 1.0);
  double before = 0.0;
  for (int j = 0; j < 64; ++j) {
    const int idj = __shfl(id, j);
    const double wj = __shfl(wk, j);
    if (idj < id) before += wj;
  }
  if (wk > 0.0 && before <= t && t < before + wk) a.out[b] = id;
}

// Second launch, for rows with no top-k limit and either no top-p limit or
// top-p alone: every chunk's weight sum against the row's max (from the
// first launch's chunk maxima); then, in the last workgroup of the row to
// arrive, with no limit, the chunk holding the draw target and the walk
// through it in id order; with top-p, the total weight gives the target,
// and if the row's first 64 tokens (merged from the first launch's chunk
// lists) reach it, the cut and the draw are taken over them in one wave,
// else the third launch takes the row.
__global__ __launch_bounds__(kSampleThreads) void sample_sum_kernel(SampleArgs a) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ SampleSmem sm;
  __shared__ double s_run[kSampleWaves];
  __shared__ unsigned s_flag;
  __shared__ double s_sums[kMaxSampleChunks];
  __shared__ int s_chunk;
  __shared__ double s_t;
  __shared__ int s_whole;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.G, b = blockIdx.x / G, g = blockIdx.x % G;
  const int V = a.V;
  const float T = a.temperature[b];
  const int k = a.top_k[b];
  const float p = a.top_p[b];
  if (!(T > 0.f) || p <= 0.f || k == 1 || !(k <= 0 || k >= V)) return;
  const bool topp = p < 1.f;
  float u = a.uniform[b];
  if (!(u >= 0.f)) u = 0.f;

  // the row's max: the chunk maxima, written by the first launch
  float M = -INFINITY;
  for (int w = 0; w < G; ++w) M = fmaxf(M, a.part_max[(size_t)b * G + w]);
  auto weight = [&](float l) { return floor((double)expf((l - M) / T) * 4294967296.0); };

  const int c0 = g * a.C, n = max(0, min(a.C, V - c0));
  const float* row = a.logits + (size_t)b * V;
  const f32x4* src = reinterpret_cast<const f32x4*>(row + c0);
  double mine = 0.0;
  if (topp) {
    // the chunk's weight per top key byte too, added into the row's
    // histogram (exact: integers below 2^53), for a nucleus beyond the
    // first 64 tokens
    for (int j = tid; j < 256; j += kSampleThreads) sm.mass[j] = 0.0;
    __syncthreads();
    for (int j0 = 0; j0 < n / 4; j0 += kSampleThreads) {
      const int j = j0 + tid;
      const f32x4 v = j < n / 4 ? src[j] : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double w = j < n / 4 ? weight(v[e]) : 0.0;
        mine += w;
        hist_add(sm, sample_key(v[e]) >> 24, w, w > 0.0);
      }
    }
    __syncthreads();
    for (int j = tid; j < 256; j += kSampleThreads)
      if (sm.mass[j] != 0.0) atomicAdd(a.row_hist + (size_t)b * 256 + j, sm.mass[j]);
  } else {
    for (int j = tid; j < n / 4; j += kSampleThreads) {
      const f32x4 v = src[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) mine += weight(v[e]);
    }
  }
  const double S = block_sum(mine, sm);
  const size_t slot = (size_t)b * G + g;
  if (tid == 0) __hip_atomic_store(a.part_sum + slot, S, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  unsigned* const cnt = a.counters2 + (size_t)b * kCntStride;
  if (!arrive_last(cnt, (unsigned)G, &s_flag)) return;
  for (int w = tid; w < G; w += kSampleThreads)  // every chunk sum in one round trip
    s_sums[w] = __hip_atomic_load(a.part_sum + (size_t)b * G + w, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (tid == 0) reset_counter(cnt);
  double R = 0.0;
  for (int w = 0; w < G; ++w) R += s_sums[w];

  if (topp) {
    // the row's first 64 tokens in rank order from the chunk lists
    const u64* lst = a.cand + (size_t)b * G * 64;
    u64* const cl = reinterpret_cast<u64*>(dyn);
    for (int i = tid; i < G * 64; i += kSampleThreads)
      cl[i] = __hip_atomic_load(lst + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    merge_lists(cl, G);
    if (wave == 0) {
      const u64 c = cl[lane];
      const bool in = c != 0ull;
      const int id = (int)(0xffffffffu - (unsigned)c);
      const double w = in ? weight(key_value((unsigned)(c >> 32))) : 0.0;
      double incl = w;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const double o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
      }
      const double target = ceil((double)p * R);
      const unsigned long long hit = __ballot(in && incl >= target);
      if (lane == 0) s_whole = hit ? 0 : 1;
      if (hit) {
        const int nkeep = __ffsll((long long)hit);
        const double wk = lane < nkeep ? w : 0.0;
        double Rk = wk;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) Rk += __shfl_xor(Rk, m);
        const double t = fmin(floor((double)u * Rk), Rk - 1.0);
        double before = 0.0;
        for (int j = 0; j < 64; ++j) {
          const int idj = __shfl(id, j);
          const double wj = __shfl(wk, j);
          if (idj < id) before += wj;
        }
        if (wk > 0.0 && before <= t && t < before + wk) a.out[b] = id;
      }
    }
    __syncthreads();
    // a nucleus beyond the first 64 tokens: the third launch takes the row
    // (and clears the row's top-byte histogram when done); else the
    // histogram is cleared here for the next call
    if (tid == 0) a.row_flag[b] = s_whole;
    if (!s_whole)
      for (int j = tid; j < 256; j += kSampleThreads)
        __hip_atomic_store(a.row_hist + (size_t)b * 256 + j, 0.0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  if (tid == 0) {
    const double t = fmin(floor((double)u * R), R - 1.0);
    double run = 0.0;
    int gc = G - 1;
    for (int w = 0; w < G; ++w) {
      if (t < run + s_sums[w]) { gc = w; break; }
      run += s_sums[w];
    }
    s_chunk = gc;
    s_t = t - run;  // the target inside that chunk
  }
  __syncthreads();
  // walk chunk s_chunk in id order: threads own consecutive runs of logits
  const int cg = s_chunk, cc0 = cg * a.C, cn = max(0, min(a.C, V - cc0));
  const double tt = s_t;
  const int per = (cn + kSampleThreads - 1) / kSampleThreads;
  const int lo = min(cn, tid * per), hi = min(cn, lo + per);
  double own = 0.0;
  for (int i = lo; i < hi; ++i) own += weight(row[cc0 + i]);
  double inc = own;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == 63) s_run[wave] = inc;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave; ++w) base += s_run[w];
  double run = base + inc - own;
  if (run <= tt && tt < run + own) {
    for (int i = lo; i < hi; ++i) {
      run += weight(row[cc0 + i]);
      if (tt < run) { a.out[b] = cc0 + i; break; }
    }
  }
}

// Third launch, for the rows the first two leave: top-p without a top-k
// limit whose nucleus the row's first 64 tokens do not reach (row_flag, set
// by the second launch), and top-k above kFastTopK (with or without
// top-p).  All G workgroups of the row select together, each on its chunk
// (loaded into LDS once), with a barrier between the steps (the row's
// workgroups are consecutive and dispatched in order, so a waiting one only
// waits for running ones; every wait is bounded):
//   a cut key by radix selection: each chunk adds its count or weight per
//   digit, among the tokens that match the digits fixed so far, into the
//   row's histogram for that byte, then every workgroup picks the same bin
//   (for top-p alone the top byte comes from the second launch's row
//   histogram);
//   the cut id among the tokens of the cut key, in id order: each chunk's
//   sum at that key, then the chunk holding the target walks its tokens;
//   top-k first (by count), then top-p among the top k (by weight, the
//   total from the first weight histogram); the draw among the kept tokens
//   in id order, the same way.
// The same definitions as the one-workgroup paths, so the same token.
// Every value that crosses workgroups is written with agent-scope stores or
// atomics.  The last workgroup to finish clears the row's histograms and
// counter.
constexpr unsigned kSampleSpin = 1u << 22;
__global__ __launch_bounds__(kSampleThreads) void sample_nucleus_kernel(SampleArgs a) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ SampleSmem sm;
  __shared__ double s_sums[kMaxSampleChunks];
  __shared__ double s_total;
  __shared__ unsigned s_flag;
  const int tid = threadIdx.x;
  const int G = a.G, b = blockIdx.x / G, g = blockIdx.x % G;
  const int V = a.V;
  const float T = a.temperature[b];
  const int k = a.top_k[b];
  const float p = a.top_p[b];
  if (!(T > 0.f) || p <= 0.f || k == 1) return;  // greedy
  const bool use_k = k > kFastTopK && k < V;
  const bool use_p = p < 1.f;
  if (use_k) {
    // top-k above the first launch's lists
  } else if (k > 1 && k <= kFastTopK) {
    return;  // the first launch's lists
  } else if (!use_p || a.row_flag[b] == 0) {
    return;  // no limit, or a nucleus within the first 64 tokens
  }
  float u = a.uniform[b];
  if (!(u >= 0.f)) u = 0.f;

  // the row's max, from the first launch
  float M = -INFINITY;
  for (int w = 0; w < G; ++w) M = fmaxf(M, a.part_max[(size_t)b * G + w]);
  auto weight = [&](float l) { return floor((double)expf((l - M) / T) * 4294967296.0); };

  // the chunk into LDS; thread t owns its consecutive tokens [lo, hi), so
  // that thread order is id order
  float* const xs = reinterpret_cast<float*>(dyn);
  const int c0 = g * a.C, n = max(0, min(a.C, V - c0));
  const f32x4* src = reinterpret_cast<const f32x4*>(a.logits + (size_t)b * V + c0);
  for (int j = tid; j < n / 4; j += kSampleThreads) reinterpret_cast<f32x4*>(xs)[j] = src[j];
  const int per = (n + kSampleThreads - 1) / kSampleThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  if (g == 0 && tid < 2)  // (if no chunk finds a cut)
    __hip_atomic_store(a.row_cut + 2 * b + tid, V - 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();

  unsigned* const cnt = a.counters3 + (size_t)b * kCntStride;
  double* const hist = a.pass_hist + (size_t)b * kPassHists * 256;
  unsigned phase = 0;
  auto row_barrier = [&]() {  // every workgroup of the row past the same point
    ++phase;
    stores_done();
    __syncthreads();
    if (tid == 0) {
      __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      poll_counter(cnt, phase * (unsigned)G, a.dev_flags, kSampleSpin);
    }
    __syncthreads();
  };
  // the row's G chunk values at sums into s_sums; returns those before chunk g
  auto gather = [&](const double* sums) {
    for (int w = tid; w < G; w += kSampleThreads)
      s_sums[w] = __hip_atomic_load(sums + (size_t)b * G + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    double before = 0.0;
    for (int w = 0; w < g; ++w) before += s_sums[w];
    return before;
  };
  // a global histogram into sm.mass
  auto load_hist = [&](const double* h) {
    for (int j = tid; j < 256; j += kSampleThreads)
      sm.mass[j] = __hip_atomic_load(h + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  };
  // one radix pass: the row's histogram of unit(l) per digit at `shift`
  // among the chunk's tokens i with (key & mask) == prefix and in(i), built
  // in global slot `slot`, then in sm.mass
  auto pass_hist = [&](int slot, int shift, unsigned prefix, unsigned mask, auto&& in,
                       auto&& unit) {
    for (int j = tid; j < 256; j += kSampleThreads) sm.mass[j] = 0.0;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += kSampleThreads) {  // (wave-uniform bounds for hist_add)
      const int i = i0 + tid;
      const float l = i < n ? xs[i] : -INFINITY;
      const unsigned key = sample_key(l);
      const bool on = i < n && (key & mask) == prefix && in(i);
      hist_add(sm, (key >> shift) & 255u, on ? unit(l) : 0.0, on);
    }
    __syncthreads();
    double* const rh = hist + (size_t)slot * 256;
    for (int j = tid; j < 256; j += kSampleThreads)
      if (sm.mass[j] != 0.0) atomicAdd(rh + j, sm.mass[j]);  // exact: integers below 2^53
    row_barrier();
    load_hist(rh);
  };
  // pick the bin at `shift` (sm.mass holds that byte's histogram) and go on
  // to the lower bytes; returns the cut key, leaves in sm.need what remains
  // to take among its tokens
  auto select = [&](int slot, int shift, unsigned prefix, unsigned mask, double need, auto&& in,
                    auto&& unit) {
    for (;;) {
      if (tid < 64) pick_bin(sm, prefix, shift, need);
      __syncthreads();
      prefix = sm.key;
      need = sm.need;
      mask |= 255u << shift;
      if (shift == 0) return prefix;
      shift -= 8;
      pass_hist(slot++, shift, prefix, mask, in, unit);
    }
  };
  // the cut id: the token of key kc, in id order among those with in(i), at
  // which the running unit(l) reaches need; into row_cut[2b + which]
  auto cut_id = [&](unsigned kc, double need, int which, auto&& in, auto&& unit) {
    double mine = 0.0;
    for (int i = lo; i < hi; ++i)
      if (sample_key(xs[i]) == kc && in(i)) mine += unit(xs[i]);
    const double Sg = block_sum(mine, sm);
    if (tid == 0)
      __hip_atomic_store(a.part_sum2 + (size_t)b * G + g, Sg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    row_barrier();
    const double before = gather(a.part_sum2);
    if (before < need && need <= before + Sg) {  // (uniform over the workgroup)
      double run = before + block_exclusive(mine, sm);
      if (run < need && need <= run + mine)
        for (int i = lo; i < hi; ++i)
          if (sample_key(xs[i]) == kc && in(i)) {
            run += unit(xs[i]);
            if (run >= need) {
              __hip_atomic_store(a.row_cut + 2 * b + which, c0 + i, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
          }
    }
    row_barrier();
    return __hip_atomic_load(a.row_cut + 2 * b + which, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto all = [](int) { return true; };
  auto count = [](float) { return 1.0; };

  // --- top-k: the k first tokens in rank order (key, then id)
  unsigned kk = 0u;
  int ik = V;
  auto in_k = [&](int i) {
    const unsigned key = sample_key(xs[i]);
    return key > kk || (key == kk && c0 + i <= ik);
  };
  if (use_k) {
    pass_hist(0, 24, 0u, 0u, all, count);
    kk = select(1, 24, 0u, 0u, (double)k, all, count);
    ik = cut_id(kk, sm.need, 0, all, count);
  }

  // --- top-p among them: the shortest rank-order prefix whose weight
  // reaches ceil(p * their total)
  unsigned kp = 0u;
  int ip = V;
  if (use_p) {
    if (use_k) {
      pass_hist(4, 24, 0u, 0u, in_k, weight);
      if (tid < 64) {  // their total, from the histogram
        double t4 = 0.0;
        for (int e = 0; e < 4; ++e) t4 += sm.mass[4 * tid + e];
        for (int m = 32; m >= 1; m >>= 1) t4 += __shfl_xor(t4, m);
        if (tid == 0) s_total = t4;
      }
      __syncthreads();
      kp = select(5, 24, 0u, 0u, ceil((double)p * s_total), in_k, weight);
    } else {
      double R = 0.0;  // the row's total, from the second launch
      for (int w = 0; w < G; ++w) R += a.part_sum[(size_t)b * G + w];
      load_hist(a.row_hist + (size_t)b * 256);
      kp = select(0, 24, 0u, 0u, ceil((double)p * R), all, weight);
    }
    ip = cut_id(kp, sm.need, 1, in_k, weight);
  }

  // --- the draw among the kept tokens, in id order
  auto kept = [&](int i) {
    const unsigned key = sample_key(xs[i]);
    return in_k(i) && (key > kp || (key == kp && c0 + i <= ip));
  };
  double mine = 0.0;
  for (int i = lo; i < hi; ++i)
    if (kept(i)) mine += weight(xs[i]);
  const double Sg = block_sum(mine, sm);
  if (tid == 0)
    __hip_atomic_store(a.part_sum3 + (size_t)b * G + g, Sg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  row_barrier();
  const double before = gather(a.part_sum3);
  double Rk = 0.0;
  for (int w = 0; w < G; ++w) Rk += s_sums[w];
  const double t = fmin(floor((double)u * Rk), Rk - 1.0);
  if (before <= t && t < before + Sg) {  // (uniform over the workgroup)
    double run = before + block_exclusive(mine, sm);
    if (run <= t && t < run + mine)
      for (int i = lo; i < hi; ++i)
        if (kept(i)) {
          run += weight(xs[i]);
          if (t < run) { a.out[b] = c0 + i; break; }
        }
  }

  // --- the last workgroup out clears the row's histograms and counter
  stores_done();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flag = prev + 1 == (phase + 1) * (unsigned)G ? 1u : 0u;
  }
  __syncthreads();
  if (s_flag != 0u) {
    for (int j = tid; j < (1 + kPassHists) * 256; j += kSampleThreads) {
      double* hp = j < 256 ? a.row_hist + (size_t)b * 256 + j : hist + (j - 256);
      __hip_atomic_store(hp, 0.0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) reset_counter(cnt);
  }
}

void sample_split(int V, int* G, int* C) {
  int g = (V + kSampleChunk - 1) / kSampleChunk;
  if (g < 1) g = 1;
  *G = g;
  *C = ((V + g - 1) / g + 3) / 4 * 4;
}

hipError_t launch_sample(const SampleArgs& a, int B, hipStream_t s) {
  const size_t lds = (size_t)a.C * 4;
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_kernel, dim3(B * a.G), dim3(kSampleThreads), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sample_sum_kernel, dim3(B * a.G), dim3(kSampleThreads),
                     (size_t)a.G * 64 * sizeof(unsigned long long), s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sample_nucleus_kernel, dim3(B * a.G), dim3(kSampleThreads), lds, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ no-allocation entry point

// qd_sample_noalloc runs the same three launches with its scratch in one
// file-scope device array instead of a handle's buffers, so that callers
// that cannot allocate (code under graph capture, tight serving loops) can
// sample.  The array is sized for batch <= kNoAllocBatch and vocab <=
// kNoAllocVocab and carved at fixed 256-byte aligned offsets (strides of the
// largest batch and chunk count).  Each GPU holds its own copy until the
// process ends; in host code its address is taken once per device with
// hipGetSymbolAddress (the array's name is not a device address there).
constexpr int kNoAllocBatch = 64;
constexpr int kNoAllocVocab = 262144;
constexpr int kNoAllocChunks = (kNoAllocVocab + kSampleChunk - 1) / kSampleChunk;
constexpr size_t na_align(size_t x) { return (x + 255) / 256 * 256; }
constexpr size_t kNaSlots = (size_t)kNoAllocBatch * kNoAllocChunks;
constexpr size_t kNaMax = 0;                                             // float [B][G]
constexpr size_t kNaIdx = kNaMax + na_align(kNaSlots * 4);               // int [B][G]
constexpr size_t kNaCand = kNaIdx + na_align(kNaSlots * 4);              // u64 [B][G][64]
constexpr size_t kNaSum = kNaCand + na_align(kNaSlots * 64 * 8);         // double [B][G]
constexpr size_t kNaSum2 = kNaSum + na_align(kNaSlots * 8);              // double [B][G]
constexpr size_t kNaSum3 = kNaSum2 + na_align(kNaSlots * 8);             // double [B][G]
constexpr size_t kNaFlag = kNaSum3 + na_align(kNaSlots * 8);             // int [B]
constexpr size_t kNaCut = kNaFlag + na_align((size_t)kNoAllocBatch * 4);  // int [B][2]
// (counters and row histograms of all three launches are contiguous: one
// fill clears them at the start of every call)
constexpr size_t kNaCnt = kNaCut + na_align((size_t)kNoAllocBatch * 2 * 4);  // u32 [B][kCntStride]
constexpr size_t kNaCnt2 = kNaCnt + na_align((size_t)kNoAllocBatch * kCntStride * 4);
constexpr size_t kNaCnt3 = kNaCnt2 + na_align((size_t)kNoAllocBatch * kCntStride * 4);
constexpr size_t kNaHist = kNaCnt3 + na_align((size_t)kNoAllocBatch * kCntStride * 4);
constexpr size_t kNaPassHist = kNaHist + na_align((size_t)kNoAllocBatch * 256 * 8);
constexpr size_t kNaBytes = kNaPassHist + na_align((size_t)kNoAllocBatch * kPassHists * 256 * 8);  // ~2.2 MB

static __device__ __align__(256) unsigned char scratch[kNaBytes];

__global__ __launch_bounds__(256) void zero_words_kernel(unsigned* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_na_mutex;
unsigned char* g_na_ptr[kMaxDevices];

// The device address of this device's copy of `scratch` (looked up once per
// device, with the device current), or null with the error in *e.
unsigned char* noalloc_scratch(int dev, hipError_t* e) {
  std::lock_guard<std::mutex> lock(g_na_mutex);
  if (g_na_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    *e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*e != hipSuccess) return nullptr;
    g_na_ptr[dev] = static_cast<unsigned char*>(ptr);
  }
  return g_na_ptr[dev];
}
}  // namespace

}  // namespace qd

extern "C" int qd_sample_noalloc(int32_t batch, int32_t vocab, const float* logits,
                                 const float* temperature, const int32_t* top_k,
                                 const float* top_p, const float* uniform, int32_t* out_ids,
                                 void* hip_stream) {
  using namespace qd;
  if (!logits || !temperature || !top_k || !top_p || !uniform || !out_ids)
    return set_global_error(QD_EINVAL, "qd_sample_noalloc: NULL pointer");
  if (reinterpret_cast<uintptr_t>(logits) % 16)
    return set_global_error(QD_EINVAL, "qd_sample_noalloc: logits must be 16-byte aligned");
  if (batch < 1 || batch > kNoAllocBatch)
    return set_global_error(QD_EINVAL,
                            "qd_sample_noalloc: batch must be in 1..64 (the static scratch's limit)");
  if (vocab < 64 || vocab > kNoAllocVocab)
    return set_global_error(QD_EINVAL,
                            "qd_sample_noalloc: vocab must be in 64..262144 (the static scratch's limit)");
  int G = 1, C = 0;
  sample_split(vocab, &G, &C);
  if ((size_t)G * 512 > (size_t)C * 4)  // the merge reuses a chunk's LDS
    return set_global_error(QD_EUNSUPPORTED, "qd_sample_noalloc: vocab too small to chunk");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_global_error(QD_EHIP, "qd_sample_noalloc: no usable current device");
  unsigned char* p = noalloc_scratch(dev, &e);
  if (p == nullptr)
    return set_global_error(QD_EHIP, std::string("qd_sample_noalloc: hipGetSymbolAddress: ") +
                                         hipGetErrorString(e));
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  // counters and row histograms start at zero in every call (a fill kernel,
  // so the call can be captured into a graph)
  hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, s,
                     reinterpret_cast<unsigned*>(p + kNaCnt), (kNaBytes - kNaCnt) / 4);
  e = hipGetLastError();
  if (e != hipSuccess)
    return set_global_error(QD_EHIP, std::string("qd_sample_noalloc: ") + hipGetErrorString(e));
  SampleArgs a{logits, vocab, temperature, top_k, top_p, uniform, out_ids, G, C,
               reinterpret_cast<float*>(p + kNaMax), reinterpret_cast<int*>(p + kNaIdx),
               reinterpret_cast<unsigned long long*>(p + kNaCand),
               reinterpret_cast<unsigned*>(p + kNaCnt), reinterpret_cast<double*>(p + kNaSum),
               reinterpret_cast<unsigned*>(p + kNaCnt2), reinterpret_cast<double*>(p + kNaHist),
               reinterpret_cast<double*>(p + kNaPassHist), reinterpret_cast<double*>(p + kNaSum2),
               reinterpret_cast<double*>(p + kNaSum3), reinterpret_cast<unsigned*>(p + kNaCnt3),
               reinterpret_cast<int*>(p + kNaFlag), reinterpret_cast<int*>(p + kNaCut), nullptr};
  e = launch_sample(a, batch, s);
  if (e != hipSuccess)
    return set_global_error(QD_EHIP, std::string("qd_sample_noalloc: ") + hipGetErrorString(e));
  return QD_OK;
}
