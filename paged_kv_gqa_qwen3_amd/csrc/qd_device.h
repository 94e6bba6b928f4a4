// Device-side building blocks of the decode step (included by the kernel
// translation units): helpers, the work-item functions and the wait used by
// the batch-1 streaming step kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>

#include "qd.h"
#include "qd_internal.h"

namespace qd {


typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ unsigned short f2bf(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// OCP E4M3, the element of an 8-bit KV pool: 1 sign, 4 exponent bits (bias
// 7), 3 mantissa bits, no infinities, NaN = S.1111.111, largest finite 448.
// Encoding rounds to nearest even and saturates at +-448; NaN encodes as 0x7F.
__device__ __forceinline__ unsigned f2e4m3(float x) {
  const unsigned u = __float_as_uint(x);
  const unsigned sign = (u >> 24) & 0x80u;
  const unsigned a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;          // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |x| >= 448, inf included: saturate
  if (a < 0x3c800000u)                        // |x| < 2^-6: subnormal steps of 2^-9
    return sign | (unsigned)rintf(__uint_as_float(a) * 512.f);  // 0..8 (8 = 2^-6)
  // normal: the 23-bit mantissa rounded to 3 bits, ties to even (a carry
  // into the exponent gives the next binade, as it should)
  const unsigned r = a + 0x7ffffu + ((a >> 20) & 1u);
  return sign | ((r >> 20) - (120u << 3));
}

// The exact value of an E4M3 code (NaN for 0x7F / 0xFF).
__device__ __forceinline__ float e4m32f(unsigned c) {
  const unsigned sign = (c & 0x80u) << 24, em = c & 0x7fu;
  if (em == 0x7fu) return __uint_as_float(0x7fc00000u);
  if (em < 8u) return __uint_as_float(sign | __float_as_uint((float)em * 0x1p-9f));
  return __uint_as_float(sign | ((em + (120u << 3)) << 20));
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// the wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr unsigned vmcnt_imm(int n) {
  return (unsigned)(n & 15) | ((unsigned)(n >> 4) << 14) | 0x70u | 0xF00u;
}
// ... and until every LDS / scalar-memory operation is done (vmcnt at its maximum).
constexpr unsigned kLgkmZero = 15u | (3u << 14) | 0x70u;

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// makes global stores visible, and even a fence limited to LDS counts
// direct-to-LDS loads as LDS writes: both wait for every outstanding vector
// memory operation of the wave, which would drain a pipeline of such loads.
// This one waits only for the wave's own LDS reads and writes.  Tiles that
// direct-to-LDS loads bring in are handed to other waves only after each
// loading wave has waited (vmcnt) for its loads before the barrier.  The
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kLgkmZero);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// bf16 hi/lo pair of v (hi = bf16(v), lo = bf16(v - hi)), stored with agent
// scope: a consumer may run in the same launch, on another XCD.
__device__ __forceinline__ void split_hilo(float v, uint16_t* hi, uint16_t* lo, size_t i) {
  const unsigned h = f2bf(v);
  __hip_atomic_store(hi + i, (uint16_t)h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(lo + i, (uint16_t)f2bf(v - __uint_as_float(h << 16)), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Cache-policy operand of a device-scope load (sc1): the data was written by
// other workgroups of the same launch.
constexpr int kDeviceScope = 16;
// ... of a streaming load (nt): data read once, not kept in the caches.
// Direct-to-LDS weight loads sustain about 13% more HBM bandwidth with it.
constexpr int kNonTemporal = 2;
// Word 3 of a raw buffer resource (32-bit data format, no swizzle); loads
// past its size return zeros.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ void unpack8(const u32x4& w, float* f) {
  f[0] = bf_lo(w.x); f[1] = bf_hi(w.x); f[2] = bf_lo(w.y); f[3] = bf_hi(w.y);
  f[4] = bf_lo(w.z); f[5] = bf_hi(w.z); f[6] = bf_lo(w.w); f[7] = bf_hi(w.w);
}

// Element types of the paged KV pool.  Both load a token row's 8
// consecutive elements per lane (16 bytes of bf16, 8 bytes of E4M3 codes);
// unpack gives their values (an 8-bit pool's codes times its scale); encode
// rounds a value to the pool's element.
struct KvBf16 {
  using Elem = uint16_t;
  using Raw = u32x4;
  static constexpr bool kFp8 = false;
  static __device__ __forceinline__ Raw load_nt(const Elem* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  static __device__ __forceinline__ Raw zero() { return u32x4{0u, 0u, 0u, 0u}; }
  static __device__ __forceinline__ void unpack(const Raw& r, float* f, float) { unpack8(r, f); }
  static __device__ __forceinline__ Elem encode(float v, float) { return f2bf(v); }
  // 8 elements staged in LDS as 16-bit slots
  static __device__ __forceinline__ Raw from_slots(const unsigned short* e) {
    return *reinterpret_cast<const u32x4*>(e);
  }
};

struct KvFp8 {
  using Elem = uint8_t;
  using Raw = u32x2;
  static constexpr bool kFp8 = true;
  static __device__ __forceinline__ Raw load_nt(const Elem* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  }
  static __device__ __forceinline__ Raw zero() { return u32x2{0u, 0u}; }
  // (v_cvt_scalef32_pk_f32_fp8 widens two OCP E4M3 codes of a 16-bit half
  // per instruction, exactly; its scale operand is left at 1)
  static __device__ __forceinline__ void unpack(const Raw& r, float* f, float scale) {
    const f32x2 p[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.x, 1.0f, false),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.x, 1.0f, true),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.y, 1.0f, false),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.y, 1.0f, true)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = p[i].x * scale;
      f[2 * i + 1] = p[i].y * scale;
    }
  }
  static __device__ __forceinline__ Elem encode(float v, float inv_scale) {
    return (Elem)f2e4m3(v * inv_scale);
  }
  static __device__ __forceinline__ Raw from_slots(const unsigned short* e) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(e);
    return u32x2{(w.x & 0xffu) | ((w.x >> 8) & 0xff00u) | ((w.y & 0xffu) << 16) |
                     ((w.y >> 16) << 24),
                 (w.z & 0xffu) | ((w.z >> 8) & 0xff00u) | ((w.w & 0xffu) << 16) |
                     ((w.w >> 16) << 24)};
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// (value, index) maximum with the lowest index winning ties; NaN never wins.
__device__ __forceinline__ void amax_merge(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__device__ __forceinline__ void wave_amax(float& bv, int& bi) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    float v = __shfl_xor(bv, m);
    int i = __shfl_xor(bi, m);
    amax_merge(bv, bi, v, i);
  }
}

__device__ __forceinline__ void set_flag(int* flags, int bit) {
  if (flags) __hip_atomic_fetch_or(flags, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Data that crosses workgroups inside one launch (split partials, and in the
// persistent kernel every activation) is written and read with agent-scope
// relaxed atomic accesses: coherent across the XCDs' L2s on gfx950 without
// whole-cache writeback or invalidation.  A producer waits until its stores
// are acknowledged before it increments a counter, so whoever reads the
// counter's new value and then loads with agent scope sees the data.  (A
// plain __threadfence() orders the same way but costs an L2 writeback and
// invalidate per wave, measured at ~0.2 us of serialised device time per
// workgroup on MI355X.)
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_agent(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_agent(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this wave's stores are performed at agent scope.
__device__ __forceinline__ void stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Returns true in the workgroup that arrives last at `counter` (which then
// resets it for the next use).
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected,
                                            unsigned* s_flag) {
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (prev == expected - 1) ? 1u : 0u;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Completion of a stage of the streaming step kernel.  Every finished unit
// of the stage (item, row group, head or sequence) adds 1 to `counter` once
// its stores are performed; the workgroup whose increment completes the
// stage raises every workgroup's flag to `phase` (an atomic maximum, so a
// flag never goes back when two stages finish close together).  Each
// workgroup polls only its own flag, on a cache line of its own, instead of
// all of them polling one counter.  counter == nullptr: not in a persistent
// step, nothing to signal.
constexpr int kFlagStride = 32;  // unsigned words between two workgroups' flags

struct Done {
  unsigned* counter;
  unsigned target;
  unsigned phase;
  unsigned* flags;
  int nflags;
};

__device__ __forceinline__ void signal_done(const Done& d) {
  if (d.counter == nullptr) return;
  __shared__ unsigned s_last;
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(d.counter, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev + 1 == d.target ? 1u : 0u;
  }
  __syncthreads();
  if (s_last != 0u)
    for (int i = threadIdx.x; i < d.nflags; i += blockDim.x)
      __hip_atomic_fetch_max(d.flags + (size_t)i * kFlagStride, d.phase, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ Done no_done() { return Done{nullptr, 0u, 0u, nullptr, 0}; }

__device__ __forceinline__ void reset_counter(unsigned* counter) {
  st_agent(counter, 0u);
}

// Loads of data written by another workgroup: agent scope when the writer
// ran in the same launch, plain (cacheable, vectorisable) loads when it was
// an earlier launch on the stream, whose completion already made it visible.
template <bool kAgent>
__device__ __forceinline__ float ld_in(const float* p) {
  if constexpr (kAgent) return ld_agent(p);
  else return *p;
}
template <bool kAgent>
__device__ __forceinline__ f32x4 ld_in4(const float* p) {
  if constexpr (kAgent) return f32x4{ld_agent(p), ld_agent(p + 1), ld_agent(p + 2), ld_agent(p + 3)};
  else return *reinterpret_cast<const f32x4*>(p);
}

// sum_{s < n} p[s * stride] in increasing s, with the loads issued 8 at a
// time (unconditional, clamped index) so that they overlap.
template <bool kAgent = true>
__device__ __forceinline__ float sum_strided(const float* p, int n, size_t stride) {
  float sum = 0.f;
  for (int s0 = 0; s0 < n; s0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ld_in<kAgent>(p + (size_t)min(s0 + j, n - 1) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < n) sum += v[j];
  }
  return sum;
}

// Output row n, batch column b, of a kPartial GEMV with `rows` rows per
// item (partials laid out [N/rows * S][rows][B]): the sum of its S split
// partials in split order.
template <bool kAgent>
__device__ __forceinline__ float split_sum(const float* part, int S, int B, int rows, int n,
                                           int b) {
  const int rg = n / rows, r = n % rows;
  return sum_strided<kAgent>(part + ((size_t)rg * S * rows + r) * B + b, S, (size_t)rows * B);
}

// Sum of v over aligned groups of n lanes (n a power of two <= 64), in a
// fixed order; every lane of a group ends with the group's sum.
__device__ __forceinline__ float group_sum(float v, int n) {
  for (int m = 1; m < n; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Items of a standalone kernel read their inputs with plain loads (written
// by an earlier launch); the waits of the persistent kernel set kInLaunch.
struct NoWait {
  static constexpr bool kInLaunch = false;
  __device__ void operator()() const {}
};

// Bounded poll (thread 0; the workgroup then proceeds together) until the
// counter reaches target; past `limit` polls it records QD_DEV_TIMEOUT and
// gives up (the results are then invalid, but the launch drains).
__device__ __forceinline__ void poll_counter(const unsigned* c, unsigned target, int* dev_flags,
                                             unsigned limit) {
  unsigned k = 0;
  while (ld_agent(c) < target) {
    if (++k > limit) {
      set_flag(dev_flags, QD_DEV_TIMEOUT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// The wait of an item of a fused launch whose inputs come from items of the
// same launch: n completion counters (kCntStride apart) must each reach
// target.  Producers sit at lower workgroup indices, which are dispatched
// first, so a waiting workgroup only waits for running or finished ones.
struct CounterWait {
  static constexpr bool kInLaunch = true;
  const unsigned* cnt;
  int n;
  unsigned target;
  int* dev_flags;
  unsigned limit;
  __device__ void operator()() const {
    if (threadIdx.x == 0)
      for (int i = 0; i < n; ++i) poll_counter(cnt + (size_t)i * kCntStride, target, dev_flags, limit);
    __syncthreads();
  }
};


// ------------------------------------------------------------------ embedding

// x[b] = E[token_b] (exact bf16 -> fp32), read from the packed table, plus
// the sums of squares of x over each group of 16 columns (the RMSNorm of the
// first QKV projection consumes them) and, for an MFMA consumer, the bf16
// pair of x times its RMSNorm gain.
__device__ inline void embed_item(const EmbedArgs& a, const Done& done, int b) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (b == 0 && a.zero != nullptr)
    for (int i = threadIdx.x; i < a.nzero; i += blockDim.x) st_agent(a.zero + (size_t)i * kCntStride, 0u);
  int tok = a.tokens[b];
  if (tok < 0 || tok >= a.V) {
    if (threadIdx.x == 0) set_flag(a.dev_flags, QD_DEV_BAD_TOKEN);
    tok = tok < 0 ? 0 : a.V - 1;
  }
  const int KT = a.H / kTileCols;
  const int rt = tok / kTileRows, r = tok % kTileRows;
  for (int base = wave * 64; base < a.H; base += 256) {
    const int k = base + lane;
    const int kt = k / kTileCols, q = (k % kTileCols) / 8, e = k % 8;
    const uint16_t v = a.table[((size_t)rt * KT + kt) * kTileElems + (q * 16 + r) * 8 + e];
    const float xv = __uint_as_float((unsigned)v << 16);
    st_agent(a.x + (size_t)b * a.H + k, xv);
    if (a.xo_hi != nullptr) split_hilo(xv * a.xo_gain[k], a.xo_hi, a.xo_lo, (size_t)b * a.H + k);
    const float ss = group_sum(xv * xv, kSsqRows);
    if (k % kSsqRows == 0) st_agent(a.ssq_out + (size_t)(k / kSsqRows) * a.Bmax + b, ss);
  }
  signal_done(done);
}

// Maximum over n (value, index) pairs per batch column (laid out [n][Bmax],
// written in this launch), lowest index on ties.  tpc = 256/Bp threads per
// column each merge every tpc-th pair with 16 loads in flight, then the
// column's threads merge (the merge is order independent).  Returns true in
// the one thread per column b < B that holds the result.  s_tmp: 8 words of
// LDS.  Every thread of the workgroup must call it.
__device__ inline bool merge_amax(const float* val, const int* idx, int n, int B, int Bmax,
                                  float* s_tmp, float& bv, int& bi, int& b) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int Bp = B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : B <= 16 ? 16 : B <= 32 ? 32 : 64;
  const int tpc = 256 / Bp;
  b = tid / tpc;
  const int p = tid - b * tpc;
  bv = -INFINITY;
  bi = 0x7fffffff;
  if (b < B) {
    for (int g0 = p; g0 < n; g0 += 16 * tpc) {
      float v[16];
      int ix[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int g = min(g0 + j * tpc, n - 1);
        v[j] = ld_agent(val + (size_t)g * Bmax + b);
        ix[j] = ld_agent(idx + (size_t)g * Bmax + b);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) amax_merge(bv, bi, v[j], ix[j]);
    }
  }
  const int wl = tpc < 64 ? tpc : 64;
  for (int m = 1; m < wl; m <<= 1) {
    const float ov = __shfl_xor(bv, m);
    const int oi = __shfl_xor(bi, m);
    amax_merge(bv, bi, ov, oi);
  }
  if (tpc > 64) {  // a column spans several waves: merge them through LDS
    int* s_ai = reinterpret_cast<int*>(s_tmp + 4);
    __syncthreads();
    if (lane == 0) { s_tmp[wave] = bv; s_ai[wave] = bi; }
    __syncthreads();
    if (p == 0)
      for (int w2 = 1; w2 < tpc / 64; ++w2) amax_merge(bv, bi, s_tmp[wave + w2], s_ai[wave + w2]);
  }
  return p == 0 && b < B;
}

// ------------------------------------------------------------------ GEMV

// LDS of a GEMV item: s_inv [64] f32 | s_ssq [256] f32 | s_res [rows][NB] f32 |
// flag (16 B) | input slice: VALU fp32 [NB][Ks], MFMA bf16 hi [NB][Ks+8]
// then lo [NB][Ks+8].  rows: 64, or 128 for items of two row tiles per wave.
__host__ __device__ constexpr size_t gemv_head_bytes(int nb, int rows = kRowsPerGroup) {
  return 256 + 1024 + (size_t)rows * nb * 4 + 16;
}

inline size_t gemv_lds_bytes_impl(int B, int kps, int rt) {
  const int nb = gemv_nb(B);
  const size_t ks = (size_t)kps * kTileCols;
  const size_t slice = nb >= 8 ? (size_t)nb * (ks + 8) * 2 * 2 : (size_t)nb * ks * 4;
  return gemv_head_bytes(nb, rt > 4 ? rt * kTileRows : kRowsPerGroup) + slice;
}

// The end of a GEMV item once rows 0..rows-1 of s_res ([rows][NB]) hold its
// results (times 1/rms under RMSNorm): the split partials (the last split of
// a row group to arrive sums them in split order), then the epilogue.
// x_old / xo_g: a residual epilogue's old residual and the next consumer's
// gain for outputs idx = tid + 256 j (idx = b * rows + r), loaded by the
// caller while its results were reduced.  Argmax items have 64 or more rows.
template <int NB, int MODE, int kRows, class Mark>
__device__ inline void gemv_finish(const GemvArgs& a, const Done& done, int rg, int s, int rows,
                                   float* s_res, unsigned* s_flag,
                                   const float (&x_old)[(kRows * NB + 255) / 256],
                                   const float (&xo_g)[(kRows * NB + 255) / 256],
                                   const Mark& mark) {
  constexpr int kXold = (kRows * NB + 255) / 256;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int B = a.B, S = a.S;
  if constexpr (MODE == kPartial) {
    // leave the partial for the consumer, which sums the S splits itself
    float* mine = a.part + (size_t)(rg * S + s) * rows * B;
    for (int idx = tid; idx < rows * B; idx += 256) {
      const int r = idx / B, b = idx - r * B;
      st_agent(mine + idx, s_res[r * NB + b]);
    }
    mark(7);
    signal_done(done);
    return;
  }
  if (S > 1) {
    float* mine = a.part + (size_t)(rg * S + s) * rows * B;
    for (int idx = tid; idx < rows * B; idx += 256) {
      const int r = idx / B, b = idx - r * B;
      st_agent(mine + idx, s_res[r * NB + b]);
    }
    if (!arrive_last(&a.counters[(size_t)rg * kCntStride], (unsigned)S, s_flag)) return;
    mark(5);
    // sum the S partials of each output in split order; a thread keeps 4
    // outputs x 8 splits of loads in flight (indices clamped, extras unused)
    const float* all = a.part + (size_t)rg * S * rows * B;
    const int n = rows * B;
    constexpr int J = 4;
    for (int i0 = tid; i0 < n; i0 += 256 * J) {
      float acc[J];
#pragma unroll
      for (int j = 0; j < J; ++j) acc[j] = 0.f;
      for (int s0 = 0; s0 < S; s0 += 8) {
        float v[J][8];
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
          for (int k = 0; k < 8; ++k)
            v[j][k] = ld_agent(all + (size_t)min(s0 + k, S - 1) * n + min(i0 + j * 256, n - 1));
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (s0 + k < S) acc[j] += v[j][k];
      }
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int idx = i0 + j * 256;
        if (idx < n) s_res[(idx / B) * NB + idx % B] = acc[j];
      }
    }
    if (tid == 0) reset_counter(&a.counters[(size_t)rg * kCntStride]);
    __syncthreads();
    mark(6);
  }

  const int N = a.N;
  const size_t row0 = (size_t)rg * rows;
  if constexpr (MODE == kStore) {
    for (int idx = tid; idx < rows * B; idx += 256) {
      const int b = idx / rows, r = idx - b * rows;
      st_agent(a.out + (size_t)b * N + row0 + r, s_res[r * NB + b]);
    }
    mark(7);
    signal_done(done);
  } else if constexpr (MODE == kResid) {
    // new residual, its sums of squares over groups of 16 rows (a group of
    // 16 lanes never spans two batch columns), and for an MFMA consumer the
    // bf16 pair of x times the consumer's RMSNorm gain
#pragma unroll
    for (int j = 0; j < kXold; ++j) {
      const int idx = tid + j * 256;  // = b * rows + r
      const bool ok = idx < rows * B;
      const int b = idx / rows, r = idx - b * rows;
      float xv = 0.f;
      if (ok) {
        xv = x_old[j] + s_res[r * NB + b];
        st_agent(a.out + (size_t)b * N + row0 + r, xv);
        if (a.xo_hi != nullptr)
          split_hilo(xv * xo_g[j], a.xo_hi, a.xo_lo, (size_t)b * N + row0 + r);
      }
      const float ss = group_sum(xv * xv, kSsqRows);
      if (ok && r % kSsqRows == 0)
        st_agent(a.ssq_out + ((row0 + r) / kSsqRows) * a.Bmax + b, ss);
    }
    mark(7);
    signal_done(done);
  } else if constexpr (MODE == kSwiGLU) {
    // row tile j of the item: gate rows 0-7, the matching up rows 8-15
    const int half = N / 2, nch = rows / 2;
    for (int idx = tid; idx < nch * B; idx += 256) {
      const int b = idx / nch, c = idx - b * nch;
      const int j = c / 8, i = c % 8;
      const float gv = s_res[(j * 16 + i) * NB + b];
      const float uv = s_res[(j * 16 + 8 + i) * NB + b];
      const float sv = gv / (1.f + expf(-gv));
      const size_t o = (size_t)b * half + (size_t)rg * nch + c;
      st_agent(a.out + o, sv * uv);
      if (a.xo_hi != nullptr) split_hilo(sv * uv, a.xo_hi, a.xo_lo, o);
    }
    mark(7);
    signal_done(done);
  } else {  // kArgmax, rows 64 or 128
    if (a.logits != nullptr) {
      for (int idx = tid; idx < rows * B; idx += 256) {
        const int b = idx / rows, r = idx - b * rows;
        a.logits[(size_t)b * N + row0 + r] = s_res[r * NB + b];
      }
    }
    for (int b = wave; b < B; b += 4) {
      float bv = s_res[lane * NB + b];
      int bi = (int)row0 + lane;
#pragma unroll
      for (int u = 1; u < kRows / 64; ++u)  // (argmax items: rows == kRows)
        amax_merge(bv, bi, s_res[(lane + 64 * u) * NB + b], (int)row0 + lane + 64 * u);
      wave_amax(bv, bi);
      if (lane == 0) {
        st_agent(a.amax_val + (size_t)rg * a.Bmax + b, bv);
        st_agent(a.amax_idx + (size_t)rg * a.Bmax + b, bi);
      }
    }
    // two levels of "last to arrive": groups of 64 row groups, then the
    // groups (no single counter takes every row group's atomic)
    const int NRG = N / rows, gq = rg / 64, ng2 = (NRG + 63) / 64;
    const int in_group = min(64, NRG - gq * 64);
    unsigned* cnt1 = a.amax_counter + (size_t)gq * kCntStride;
    if (!arrive_last(cnt1, (unsigned)in_group, s_flag)) return;
    {
      float bv;
      int bi, b;
      if (merge_amax(a.amax_val + (size_t)gq * 64 * a.Bmax, a.amax_idx + (size_t)gq * 64 * a.Bmax,
                     in_group, B, a.Bmax, s_res, bv, bi, b)) {
        st_agent(a.amax_val2 + (size_t)gq * a.Bmax + b, bv);
        st_agent(a.amax_idx2 + (size_t)gq * a.Bmax + b, bi);
      }
    }
    if (tid == 0) reset_counter(cnt1);
    unsigned* cnt2 = a.amax_counter + (size_t)ng2 * kCntStride;
    if (!arrive_last(cnt2, (unsigned)ng2, s_flag)) return;
    {
      float bv;
      int bi, b;
      if (merge_amax(a.amax_val2, a.amax_idx2, ng2, B, a.Bmax, s_res, bv, bi, b))
        a.next_ids[b] = bi == 0x7fffffff ? -1 : bi;
    }
    if (tid == 0) reset_counter(cnt2);
  }
}

// y[b][n] = sum_k W[n][k] h[b][k], h = x or RMSNorm(x), W packed bf16.
//
// One item = rt row tiles (16 rows each) x one K slice of kps tiles.  Wave w
// works on row tile w % rt of the item and on every (4/rt)-th k-tile of the
// slice from w / rt on; with RPW = 2 (rt = 8, MFMA only) on row tiles w and
// w + 4 and every k-tile, the two tiles of one k-tile in turn, so that each
// input operand read from LDS feeds both.  It streams its tiles with one 16-byte load per lane
// per 1 KB tile and CH tiles in flight: the first CH go out before the item
// waits for its input, and each later one as soon as the registers it lands
// in are free.
//   NB = 1  : VALU path, fp32 FMA; the K slice of the input (times the
//             RMSNorm gain) is staged in LDS.
//   NB >= 8 : MFMA path, v_mfma_f32_16x16x32_bf16 with the weight tile as
//             operand A and the input as a pair of bf16 (hi = bf16(x), lo =
//             bf16(x - hi)): at NB = 8 one MFMA per tile, columns 0..7 the
//             hi halves and 8..15 the lo halves of the 8 batch columns
//             (added at the end); at NB >= 16 NB/16 blocks of 16 batch
//             columns, two MFMAs per tile: ~16 significant bits of input instead of 8
//             (bf16 inputs alone move a 36-layer model's logits by ~2% of
//             their maximum, beyond the step's 2e-2 tolerance).  The producer
//             of the input wrote the pairs once (xh, xl: [64][K] bf16, times
//             the RMSNorm gain); the item copies its K slice of them to LDS,
//             once for its 4 row tiles (reading the B operand per wave from
//             L2 instead would pass twice the weight bytes through each CU's
//             load unit at 16 columns, one row tile per item).
// Under RMSNorm each result row is scaled by 1/rms of its batch column at
// the end, so the input does not wait for the producer's sums of squares.
// Waves that share a row tile add their results in LDS in K order.  With
// S > 1 splits of K, each item writes its partial rows and the last of the
// row group's S items to arrive sums the partials in split order
// (deterministic) and runs the epilogue.
template <int NB, int MODE, int CH = kMaxTilesInFlight, class Wait, int RPW = 1>
__device__ inline void gemv_item(const GemvArgs& a, const uint16_t* w, const float* gain,
                                 const Done& done, int item, unsigned char* smem,
                                 const Wait& wait) {
#ifdef QD_STEP_TRACE
  auto mark = [&](int e) {
    if (a.trace != nullptr && threadIdx.x == 0 && item < kTraceItems)
      a.trace[(size_t)item * 8 + e] = __builtin_amdgcn_s_memrealtime();
  };
#else
  auto mark = [](int) {};
#endif
  mark(0);
  constexpr bool kMfma = NB >= 8;
  constexpr bool kSplitCols = NB == 8;  // hi and lo side by side in one operand
  constexpr bool kAgent = Wait::kInLaunch;
  constexpr int NCB = kMfma && !kSplitCols ? NB / 16 : 1;
  static_assert(RPW == 1 || (RPW == 2 && kMfma), "two row tiles per wave: MFMA items");
  constexpr int kRows = RPW * kRowsPerGroup;  // most rows of an item
  float* s_inv = reinterpret_cast<float*>(smem);
  float* s_ssq = s_inv + kMaxBatch;
  float* s_res = s_ssq + 256;
  unsigned* s_flag = reinterpret_cast<unsigned*>(s_res + kRows * NB);
  unsigned char* xs_base = smem + gemv_head_bytes(NB, kRows);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int B = a.B, S = a.S, RT = RPW == 2 ? 8 : a.rt, WS = RPW == 2 ? 1 : 4 / RT;
  const int rows = RT * kTileRows;
  const int rg = item / S, s = item - rg * S;
  const int KT = a.K / kTileCols;
  const int kt0 = s * a.kps;
  const int kt1 = min(KT, kt0 + a.kps);
  const int nk = kt1 - kt0;
  const int Ks = nk * kTileCols;
  const int tj = RPW == 2 ? wave : wave % RT, kph = RPW == 2 ? 0 : wave / RT;  // row tile, K phase
  const int nkw = kph < nk ? (nk - kph + WS - 1) / WS : 0;  // k-tiles of this wave
  const int lastw = nkw > 0 ? nkw - 1 : 0;
  const int kw0 = kt0 + min(kph, nk - 1);  // first k-tile of this wave
  const u32x4* wp = reinterpret_cast<const u32x4*>(w) +
                    ((size_t)(rg * RT + tj) * KT + kw0) * 64 + lane;

  // Loads go out in the order their data is needed, so that waiting for
  // one never waits for a later one (a wave's loads complete in issue
  // order): the input slice, the RMSNorm sums of squares, then the first CH
  // weight tiles.  When the input is produced in the same launch (kAgent:
  // a fused launch), the weight tiles go out first and the input only
  // after the wait, with device-scope loads.
  //
  // MFMA path: up to kStageLoads 16-byte pieces of the input slice per
  // thread in registers (12 pieces cost a third workgroup per CU in
  // registers: batch 8 and 16 took 3.50 and 4.22 ms per step against 3.16
  // and 3.88 with 8); further pieces are copied after the weight tiles.
  // VALU path: up to kValuPre 4-float groups of the input and of the gain.
  constexpr int kStageLoads = 8;
  constexpr int kValuPre = 2;
  const int K8 = Ks / 8, n_in = kMfma ? B * K8 : 0;
  u32x4 inb[kMfma ? kStageLoads : 1];
  auto in_src = [&](int idx) {
    const int hl = idx >= n_in, rem = idx - hl * n_in;
    const int b = rem / K8, c = (rem - b * K8) * 8;
    return (hl ? a.xl : a.xh) + (size_t)b * a.K + kt0 * kTileCols + c;
  };
  auto in_dst = [&](int idx) {
    const int hl = idx >= n_in, rem = idx - hl * n_in;
    const int b = rem / K8, c = (rem - b * K8) * 8;
    return hl * NB * (Ks + 8) + b * (Ks + 8) + c;
  };
  const int K4 = Ks / 4, n_v4 = kMfma ? 0 : B * K4;  // VALU: 4-float groups of the slice
  f32x4 xpre[kMfma ? 1 : kValuPre], gpre[kMfma ? 1 : kValuPre];
  const bool norm = a.ssq != nullptr;
  // device-scope 16-byte loads of in-launch input pieces
  const __amdgpu_buffer_rsrc_t rs_hi = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.xh), 0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rs_lo = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.xl), 0, 0x7fffffff, kBufferWord3);
  auto in_load = [&](int idx) -> u32x4 {
    if constexpr (!kAgent) return *reinterpret_cast<const u32x4*>(in_src(idx));
    const int hl = idx >= n_in, rem = idx - hl * n_in;
    const int b = rem / K8, c = (rem - b * K8) * 8;
    const int off = (b * a.K + kt0 * kTileCols + c) * 2;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hl ? rs_lo : rs_hi, off,
                                                                           0, kDeviceScope));
  };
  if constexpr (kAgent) {
    // (issued after the wait below)
  } else if constexpr (kMfma) {
#pragma unroll
    for (int j = 0; j < kStageLoads; ++j) {
      const int idx = tid + j * 256;
      if (idx < 2 * n_in) inb[j] = in_load(idx);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kValuPre; ++j) {
      const int g4 = tid + j * 256;
      if (g4 < n_v4) {
        const int b = g4 / K4, c = (g4 - b * K4) * 4;
        xpre[j] = *reinterpret_cast<const f32x4*>(a.x + (size_t)b * a.K + kt0 * kTileCols + c);
        if (norm) gpre[j] = *reinterpret_cast<const f32x4*>(gain + kt0 * kTileCols + c);
      }
    }
  }

  // RMSNorm sums of squares: one partial per 16 rows of the producer,
  // [K/16][Bmax].  Thread t adds batch column t % NB's partials t / NB,
  // t / NB + 256/NB, ... in order (kSsq loads in flight: hidden sizes up
  // to 16 * kSsq * 256/NB; beyond that the rest after the weight tiles);
  // the 256/NB parts are then added in order.
  constexpr int kParts = 256 / NB;
  constexpr int kSsq = NB >= 16 ? 16 : 8;
  const int ng = a.K / kSsqRows;
  const int sb = tid % NB, sp = tid / NB;
  float sv[kSsq];
  auto load_ssq = [&](int g0) {
#pragma unroll
    for (int j = 0; j < kSsq; ++j)
      sv[j] = ld_in<kAgent>(a.ssq + (size_t)min(g0 + j * kParts, ng - 1) * a.Bmax + min(sb, B - 1));
  };
  if (norm && !kAgent) load_ssq(sp);

  // Weight tiles: every load is issued unconditionally (tile index clamped
  // to the wave's range) so that the loads stay in flight together; only
  // compute is guarded.  Offsets in 32 bits (a wave's tiles lie within one
  // projection).
  // wave-local tile i: k-tile i (RPW 1), or k-tile i / 2 of row tile
  // tj + 4 * (i % 2) (RPW 2); nt tiles in all
  const unsigned wstep = (unsigned)WS * 64u;
  const unsigned rstep = 4u * (unsigned)KT * 64u;  // row tile w -> w + 4
  const int nt = nkw * RPW;
  auto wtile = [&](int i) {
    if constexpr (RPW == 2) return wp + (unsigned)(i & 1) * rstep + (unsigned)min(i >> 1, lastw) * wstep;
    return wp + (unsigned)min(i, lastw) * wstep;
  };
  u32x4 wbuf[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) wbuf[i] = __builtin_nontemporal_load(wtile(i));

  wait();
  mark(1);
  if constexpr (kAgent) {
    if (norm) load_ssq(sp);
    if constexpr (kMfma) {
#pragma unroll
      for (int j = 0; j < kStageLoads; ++j) {
        const int idx = tid + j * 256;
        if (idx < 2 * n_in) inb[j] = in_load(idx);
      }
    }
  }

  // Stage the input slice: MFMA, the pairs of the B live columns, hi rows
  // first, then lo rows (LDS columns B..NB-1 keep whatever they held: they
  // only feed outputs that are never stored); VALU, x times the gain.
  const int P = kMfma ? Ks + 8 : Ks;
  if constexpr (kMfma) {
    unsigned short* xs = reinterpret_cast<unsigned short*>(xs_base);
#pragma unroll
    for (int j = 0; j < kStageLoads; ++j) {
      const int idx = tid + j * 256;
      if (idx < 2 * n_in) *reinterpret_cast<u32x4*>(xs + in_dst(idx)) = inb[j];
    }
    for (int idx = tid + kStageLoads * 256; idx < 2 * n_in; idx += 256)
      *reinterpret_cast<u32x4*>(xs + in_dst(idx)) = in_load(idx);
  } else {
    const float* grow = gain + kt0 * kTileCols;
#pragma unroll
    for (int j = 0; j < kValuPre; ++j) {
      const int g4 = tid + j * 256;
      if (!kAgent && g4 < n_v4) {
        const int b = g4 / K4, c = (g4 - b * K4) * 4;
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(xs_base) + b * P + c) =
            norm ? xpre[j] * gpre[j] : xpre[j];
      }
    }
    for (int g4 = tid + (kAgent ? 0 : kValuPre * 256); g4 < n_v4; g4 += 256) {
      const int b = g4 / K4, c = (g4 - b * K4) * 4;
      f32x4 v = ld_in4<kAgent>(a.x + (size_t)b * a.K + kt0 * kTileCols + c);
      if (norm) v *= *reinterpret_cast<const f32x4*>(grow + c);
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(xs_base) + b * P + c) = v;
    }
  }
  if (norm) {
    // The first sums stay opaque until here: otherwise the compiler adds
    // the first one where it is loaded, so that the wave waits for it (and
    // for every load issued before it) before the weight tiles go out.
#pragma unroll
    for (int j = 0; j < kSsq; ++j) asm volatile("" : "+v"(sv[j]));
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kSsq; ++j) ss += sp + j * kParts < ng ? sv[j] : 0.f;
    for (int g0 = sp + kSsq * kParts; g0 < ng; g0 += kSsq * kParts) {
      load_ssq(g0);
#pragma unroll
      for (int j = 0; j < kSsq; ++j) ss += g0 + j * kParts < ng ? sv[j] : 0.f;
    }
    s_ssq[tid] = ss;
  }
  __syncthreads();
  if (norm && tid < B) {
    float ss = 0.f;
    for (int p = 0; p < kParts; ++p) ss += s_ssq[p * NB + tid];
    s_inv[tid] = rsqrtf(ss / (float)a.K + a.eps);
  }
  __syncthreads();
  mark(2);

  // Tiles are consumed in batches of KB: the batch's input operands are
  // read from LDS first, then its MFMAs (or FMAs) run on KB independent
  // accumulators, so neither the LDS round trip nor the accumulation chain
  // is paid per tile; each consumed tile's registers are refilled with the
  // tile CH ahead at once.
  constexpr int KB = kSplitCols ? 4 : kMfma ? (NCB == 1 ? 2 : 1) : 2;
  static_assert(CH % KB == 0, "whole batches of tiles in flight");
  float acc_v[KB][kMfma ? 1 : NB];
  f32x4 acc_m[KB][NCB];
#pragma unroll
  for (int q = 0; q < KB; ++q) {
#pragma unroll
    for (int b = 0; b < (kMfma ? 1 : NB); ++b) acc_v[q][b] = 0.f;
#pragma unroll
    for (int c = 0; c < NCB; ++c) acc_m[q][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // wave-local tile i is k-tile kph + WS*i of the item's slice
  const unsigned short* xsh = reinterpret_cast<const unsigned short*>(xs_base);
  const float* xsf = reinterpret_cast<const float*>(xs_base);
  struct BIn { u32x4 h[NCB], l[NCB]; f32x4 f0[NB], f1[NB]; };
  auto read_in = [&](int i, BIn& bi) {
    const int t = kph + WS * (i / RPW);
    if constexpr (kSplitCols) {
      // LDS rows 0..7 hold the hi halves, 8..15 the lo halves: operand
      // column (lane % 16) reads row lane % 16
      bi.h[0] = *reinterpret_cast<const u32x4*>(xsh + (lane & 15) * P + t * kTileCols +
                                                (lane >> 4) * 8);
    } else if constexpr (kMfma) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int off = (cb * 16 + (lane & 15)) * P + t * kTileCols + (lane >> 4) * 8;
        bi.h[cb] = *reinterpret_cast<const u32x4*>(xsh + off);
        bi.l[cb] = *reinterpret_cast<const u32x4*>(xsh + NB * P + off);
      }
    } else {
      const float* xp = xsf + t * kTileCols + (lane >> 4) * 8;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        bi.f0[b] = *reinterpret_cast<const f32x4*>(xp + b * P);
        bi.f1[b] = *reinterpret_cast<const f32x4*>(xp + b * P + 4);
      }
    }
  };
  auto mac = [&](const u32x4& wv, const BIn& bi, int q) {
    if constexpr (kSplitCols) {
      acc_m[q][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, wv), __builtin_bit_cast(bf16x8, bi.h[0]), acc_m[q][0], 0, 0, 0);
    } else if constexpr (kMfma) {
      const bf16x8 wa = __builtin_bit_cast(bf16x8, wv);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        acc_m[q][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            wa, __builtin_bit_cast(bf16x8, bi.h[cb]), acc_m[q][cb], 0, 0, 0);
        acc_m[q][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            wa, __builtin_bit_cast(bf16x8, bi.l[cb]), acc_m[q][cb], 0, 0, 0);
      }
    } else {
      float wf[8];
      unpack8(wv, wf);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float acc = acc_v[q][b];
        acc = fmaf(wf[0], bi.f0[b].x, acc); acc = fmaf(wf[1], bi.f0[b].y, acc);
        acc = fmaf(wf[2], bi.f0[b].z, acc); acc = fmaf(wf[3], bi.f0[b].w, acc);
        acc = fmaf(wf[4], bi.f1[b].x, acc); acc = fmaf(wf[5], bi.f1[b].y, acc);
        acc = fmaf(wf[6], bi.f1[b].z, acc); acc = fmaf(wf[7], bi.f1[b].w, acc);
        acc_v[q][b] = acc;
      }
    }
  };
  // steady state: consume a batch, refill its registers with the tiles CH
  // ahead.  With RPW 2 a batch's tiles alternate between the two row tiles
  // (accumulator q % 2), and each pair shares one input operand.
  static_assert(KB % RPW == 0, "a batch holds both row tiles of its k-tiles");
  int c0 = 0;
  for (; c0 + CH < nt; c0 += CH) {
#pragma unroll
    for (int i0 = 0; i0 < CH; i0 += KB) {
      BIn bi[KB / RPW];
#pragma unroll
      for (int q = 0; q < KB / RPW; ++q) read_in(c0 + i0 + q * RPW, bi[q]);
#pragma unroll
      for (int q = 0; q < KB; ++q) {
        mac(wbuf[i0 + q], bi[q / RPW], q);
        wbuf[i0 + q] = __builtin_nontemporal_load(wtile(c0 + CH + i0 + q));
      }
    }
  }
#pragma unroll
  for (int i0 = 0; i0 < CH; i0 += KB) {
    if (c0 + i0 >= nt) break;
    BIn bi[KB / RPW];
#pragma unroll
    for (int q = 0; q < KB / RPW; ++q) read_in(min(c0 + i0 + q * RPW, nt - 1), bi[q]);
#pragma unroll
    for (int q = 0; q < KB; ++q)
      if (c0 + i0 + q < nt) mac(wbuf[i0 + q], bi[q / RPW], q);
  }
  // the batch accumulators, added in a fixed order (per row tile: q % RPW)
#pragma unroll
  for (int q = RPW; q < KB; ++q) {
#pragma unroll
    for (int b = 0; b < (kMfma ? 1 : NB); ++b) acc_v[q % RPW][b] += acc_v[q][b];
#pragma unroll
    for (int c = 0; c < NCB; ++c) acc_m[q % RPW][c] += acc_m[q][c];
  }

  // The residual epilogue's old residual and the next consumer's gain
  // (thread: outputs idx = tid + 256 j, idx = b * rows + r), loaded while
  // the waves' results are reduced.  Every split fetches them; only the one
  // that finishes the row group uses them.
  constexpr int kXold = (kRows * NB + 255) / 256;
  float x_old[kXold], xo_g[kXold];
  if constexpr (MODE == kResid) {
#pragma unroll
    for (int j = 0; j < kXold; ++j) {
      const int idx = tid + j * 256;
      if (idx < rows * B) {
        const size_t n = (size_t)rg * rows + idx % rows;
        x_old[j] = (a.res_in != nullptr ? a.res_in : a.out)[(size_t)(idx / rows) * a.N + n];
        xo_g[j] = a.xo_hi != nullptr ? a.xo_gain[n] : 0.f;
      }
    }
  }
  mark(3);

  // Per-wave results (times 1/rms of the batch column under RMSNorm) ->
  // s_res slot `wave` = [16 rows][NB]; then the waves of a row tile are
  // added in K order into the slot of its first wave, so that rows 0..rows-1
  // of s_res hold the item's rows.
  if constexpr (kSplitCols) {
    // column c < 8 (hi) plus its partner c + 8 (lo), lane ^ 8
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      f32x4 tot;
#pragma unroll
      for (int r = 0; r < 4; ++r) tot[r] = acc_m[u][0][r] + __shfl_xor(acc_m[u][0][r], 8);
      const int col = lane & 15;
      if (col < 8) {
        const float sc = norm && col < B ? s_inv[col] : 1.f;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s_res[((wave + 4 * u) * 16 + (lane >> 4) * 4 + r) * NB + col] = tot[r] * sc;
      }
    }
  } else if constexpr (kMfma) {
#pragma unroll
    for (int u = 0; u < RPW; ++u)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int col = cb * 16 + (lane & 15);
        const float sc = norm && col < B ? s_inv[col] : 1.f;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s_res[((wave + 4 * u) * 16 + (lane >> 4) * 4 + r) * NB + col] = acc_m[u][cb][r] * sc;
      }
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v = acc_v[0][b];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (norm && b < B) v *= s_inv[b];
      if (lane < 16) s_res[(wave * 16 + lane) * NB + b] = v;
    }
  }
  __syncthreads();
  if (WS > 1) {
    for (int idx = tid; idx < rows * NB; idx += 256) {
      float v = s_res[idx];
      for (int k = 1; k < WS; ++k) v += s_res[idx + k * rows * NB];
      s_res[idx] = v;
    }
    __syncthreads();
  }
  mark(4);

  gemv_finish<NB, MODE, kRows>(a, done, rg, s, rows, s_res, s_flag, x_old, xo_g, mark);
}

// ------------------------------------------------------------------ GEMV, 32 and 64 columns

// At 32 and 64 batch columns an item's input (the bf16 pair of every
// column) is as large per k-tile as 32 or 64 weight rows, so staging a whole
// K slice in LDS caps the slice at a few k-tiles, and the split partials
// (S x N x B floats, written and read back) then outweigh the weights.  These
// items stream their input slice through LDS in chunks of kWideChunk k-tiles
// instead, in two buffers (the next chunk loads while the current one is
// consumed), so that K is split only to give every CU work; and each wave
// owns RW row tiles (w, w + 4, ...), so that each input operand it reads
// from LDS feeds RW MFMA pairs.  Weight tiles stream one chunk ahead in
// registers.
constexpr int kWideChunk = 4;
constexpr size_t kWideHead = (size_t)(kMaxBatch + 256) * 4 + 16;  // s_inv, s_ssq, flag
__host__ __device__ constexpr size_t gemv_wide_lds_bytes(int nb, int rw) {
  // s_res [rows][nb] f32 shares the space of the two input buffers
  // [hi | lo][nb][kWideChunk * 32 + 8] bf16
  return kWideHead + ((size_t)rw * kRowsPerGroup * nb * 4 > (size_t)2 * 2 * nb * (kWideChunk * kTileCols + 8) * 2
                          ? (size_t)rw * kRowsPerGroup * nb * 4
                          : (size_t)2 * 2 * nb * (kWideChunk * kTileCols + 8) * 2);
}

// The end of a 32- or 64-column item of a row group split S > 1 ways
// (kStore, kResid, kSwiGLU).  At these widths a row group's partials are
// large (S x rows x B floats), so instead of the last split summing all of
// them, every split writes its partial, waits until all S have (the items
// of a row group are consecutive workgroups, dispatched in order, so a
// waiting split only waits for running or dispatched ones; bounded), then
// sums its 1/S share of the outputs over the S partials in split order and
// runs the epilogue on that share.  Shares are whole units of 16 outputs
// (16 rows of one batch column: an RMSNorm sum-of-squares group, or a
// gate/up row tile).  Partials are laid out [split][B][rows].
constexpr unsigned kWideSpin = 1u << 22;
template <int NB, int MODE, int kRows, class Mark>
__device__ inline void gemv_finish_coop(const GemvArgs& a, int rg, int s, const float* s_res,
                                        const Mark& mark) {
  static_assert(MODE == kStore || MODE == kResid || MODE == kSwiGLU, "splittable epilogues");
  const int tid = threadIdx.x, lane = tid & 63;
  const int B = a.B, S = a.S, N = a.N, n = kRows * B;
  float* mine = a.part + (size_t)(rg * S + s) * n;
  for (int idx = tid; idx < n; idx += 256) {
    const int b = idx / kRows, r = idx - b * kRows;
    st_agent(mine + idx, s_res[r * NB + b]);
  }
  stores_done();
  __syncthreads();
  unsigned* cnt = &a.counters[(size_t)rg * kCntStride];
  if (tid == 0) {
    __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    poll_counter(cnt, (unsigned)S, a.dev_flags, kWideSpin);
  }
  __syncthreads();
  mark(5);
  const int units = n / 16;
  const int lo = 16 * (int)((long long)units * s / S), hi = 16 * (int)((long long)units * (s + 1) / S);
  const float* all = a.part + (size_t)rg * S * n;
  const size_t row0 = (size_t)rg * kRows;
  for (int base = lo; base < hi; base += 256) {
    const int idx = base + tid;
    const bool ok = idx < hi;
    const int ic = ok ? idx : lo;
    const int b = ic / kRows, r = ic - b * kRows;
    // the S partials of this output, in split order, 8 loads in flight
    float v = 0.f;
    for (int s0 = 0; s0 < S; s0 += 8) {
      float t[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = ld_agent(all + (size_t)min(s0 + k, S - 1) * n + ic);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (s0 + k < S) v += t[k];
    }
    if constexpr (MODE == kStore) {
      if (ok) st_agent(a.out + (size_t)b * N + row0 + r, v);
    } else if constexpr (MODE == kResid) {
      float xv = 0.f;
      if (ok) {
        xv = (a.res_in != nullptr ? a.res_in : a.out)[(size_t)b * N + row0 + r] + v;
        st_agent(a.out + (size_t)b * N + row0 + r, xv);
        if (a.xo_hi != nullptr)
          split_hilo(xv * a.xo_gain[row0 + r], a.xo_hi, a.xo_lo, (size_t)b * N + row0 + r);
      }
      const float ss = group_sum(xv * xv, kSsqRows);
      if (ok && r % kSsqRows == 0) st_agent(a.ssq_out + ((row0 + r) / kSsqRows) * a.Bmax + b, ss);
    } else {  // kSwiGLU: rows 0-7 of a 16-row unit are gate channels, 8-15 the matching up ones
      const float uv = __shfl(v, (lane & ~15) + 8 + (lane & 7));
      if (ok && (r & 15) < 8) {
        const int c = (r >> 4) * 8 + (r & 7);
        const float sv = v / (1.f + expf(-v));
        const size_t o = (size_t)b * (N / 2) + (size_t)rg * (kRows / 2) + c;
        st_agent(a.out + o, sv * uv);
        if (a.xo_hi != nullptr) split_hilo(sv * uv, a.xo_hi, a.xo_lo, o);
      }
    }
  }
  mark(6);
  // every split has passed its wait once all have arrived a second time:
  // the last one resets the counter for the next launch
  stores_done();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1 == 2u * (unsigned)S) reset_counter(cnt);
  }
  mark(7);
}

template <int NB, int MODE, int RW>
__device__ inline void gemv_wide_item(const GemvArgs& a, const Done& done, int item,
                                      unsigned char* smem) {
#ifdef QD_STEP_TRACE
  auto mark = [&](int e) {
    if (a.trace != nullptr && threadIdx.x == 0 && item < kTraceItems)
      a.trace[(size_t)item * 8 + e] = __builtin_amdgcn_s_memrealtime();
  };
#else
  auto mark = [](int) {};
#endif
  mark(0);
  static_assert(NB == 16 || NB == 32 || NB == 64, "16, 32 or 64 batch columns");
  constexpr int NCB = NB / 16;             // 16-column blocks
  constexpr int kRows = RW * kRowsPerGroup;
  constexpr int C = kWideChunk;
  constexpr int P = C * kTileCols + 8;     // LDS row of one column's chunk (bf16, padded)
  constexpr int CH = C * RW;               // weight tiles in flight per wave: one chunk
  constexpr int QPC = C * kTileCols / 8;   // 16-byte pieces of one column's chunk
  constexpr int kPieces = 2 * NB * QPC / 256;  // input pieces per thread per chunk
  float* s_inv = reinterpret_cast<float*>(smem);
  float* s_ssq = s_inv + kMaxBatch;
  unsigned* s_flag = reinterpret_cast<unsigned*>(s_ssq + 256);
  unsigned char* body = smem + kWideHead;
  float* s_res = reinterpret_cast<float*>(body);
  unsigned short* xb = reinterpret_cast<unsigned short*>(body);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int B = a.B, S = a.S;
  const int rg = item / S, s = item - rg * S;
  const int KT = a.K / kTileCols;
  const int kt0 = s * a.kps, kt1 = min(KT, kt0 + a.kps), nk = kt1 - kt0;
  const int nch = (nk + C - 1) / C;
  const bool norm = a.ssq != nullptr;

  // input chunk c: pieces idx = tid + 256 j -> (hi|lo, column b, piece q)
  u32x4 inr[kPieces];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int idx = tid + j * 256;
      const int hl = idx / (NB * QPC), rem = idx - hl * (NB * QPC);
      const int b = rem / QPC, q = rem - b * QPC;
      const int k = (kt0 + c * C) * kTileCols + q * 8;
      if (b < B && k < kt1 * kTileCols)
        inr[j] = *reinterpret_cast<const u32x4*>((hl ? a.xl : a.xh) + (size_t)b * a.K + k);
    }
  };
  auto store_chunk = [&](int c) {
    unsigned short* buf = xb + (c & 1) * 2 * NB * P;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int idx = tid + j * 256;
      const int hl = idx / (NB * QPC), rem = idx - hl * (NB * QPC);
      const int b = rem / QPC, q = rem - b * QPC;
      const int k = (kt0 + c * C) * kTileCols + q * 8;
      if (b < B && k < kt1 * kTileCols)
        *reinterpret_cast<u32x4*>(buf + hl * NB * P + b * P + q * 8) = inr[j];
    }
  };

  // weight tile i of this wave: k-tile i / RW of the slice, row tile
  // wave + 4 * (i % RW) of the item (indices past the slice repeat its last
  // tile: every load is issued, compute is guarded)
  const u32x4* wp = reinterpret_cast<const u32x4*>(a.w) +
                    ((size_t)(rg * 4 * RW + wave) * KT + kt0) * 64 + lane;
  const unsigned rstep = 4u * (unsigned)KT * 64u;
  const int nt = nk * RW;
  auto wtile = [&](int i) {
    const int ii = min(i, nt - 1);
    return wp + (unsigned)(ii % RW) * rstep + (unsigned)(ii / RW) * 64u;
  };

  // loads in the order their data is needed: chunk 0 of the input, the
  // RMSNorm sums of squares, the first chunk's weight tiles
  load_chunk(0);
  constexpr int kParts = 256 / NB;
  constexpr int kSsq = 16;
  const int ng = a.K / kSsqRows;
  const int sb = tid % NB, sp = tid / NB;
  float sv[kSsq];
  auto load_ssq = [&](int g0) {
#pragma unroll
    for (int j = 0; j < kSsq; ++j)
      sv[j] = a.ssq[(size_t)min(g0 + j * kParts, ng - 1) * a.Bmax + min(sb, B - 1)];
  };
  if (norm) load_ssq(sp);
  u32x4 wbuf[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) wbuf[i] = __builtin_nontemporal_load(wtile(i));
  mark(1);
  store_chunk(0);
  if (norm) {
    // The first sums stay opaque until here: otherwise the compiler adds
    // the first one where it is loaded, so that the wave waits for it (and
    // for every load issued before it) before the weight tiles go out.
#pragma unroll
    for (int j = 0; j < kSsq; ++j) asm volatile("" : "+v"(sv[j]));
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kSsq; ++j) ss += sp + j * kParts < ng ? sv[j] : 0.f;
    for (int g0 = sp + kSsq * kParts; g0 < ng; g0 += kSsq * kParts) {
      load_ssq(g0);
#pragma unroll
      for (int j = 0; j < kSsq; ++j) ss += g0 + j * kParts < ng ? sv[j] : 0.f;
    }
    s_ssq[tid] = ss;
  }
  __syncthreads();
  if (norm && tid < B) {
    float ss = 0.f;
    for (int p = 0; p < kParts; ++p) ss += s_ssq[p * NB + tid];
    s_inv[tid] = rsqrtf(ss / (float)a.K + a.eps);
  }
  mark(2);

  f32x4 acc[RW][NCB];
#pragma unroll
  for (int u = 0; u < RW; ++u)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[u][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this lane's input operand of k-tile tt of a chunk buffer: column
  // cb * 16 + lane % 16, k-group lane / 16
  auto mac_tile = [&](const unsigned short* buf, int tt) {
    u32x4 h[NCB], l[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int off = (cb * 16 + (lane & 15)) * P + tt * kTileCols + (lane >> 4) * 8;
      h[cb] = *reinterpret_cast<const u32x4*>(buf + off);
      l[cb] = *reinterpret_cast<const u32x4*>(buf + NB * P + off);
    }
#pragma unroll
    for (int u = 0; u < RW; ++u) {
      const bf16x8 wa = __builtin_bit_cast(bf16x8, wbuf[tt * RW + u]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        acc[u][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, __builtin_bit_cast(bf16x8, h[cb]),
                                                             acc[u][cb], 0, 0, 0);
        acc[u][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, __builtin_bit_cast(bf16x8, l[cb]),
                                                             acc[u][cb], 0, 0, 0);
      }
    }
  };
  // every chunk but the last is whole: consume it while the next one's
  // input loads and its weight tiles replace the consumed ones
  int c = 0;
  for (; c + 1 < nch; ++c) {
    __syncthreads();  // chunk c is in its buffer; the other buffer is free
    load_chunk(c + 1);
    const unsigned short* buf = xb + (c & 1) * 2 * NB * P;
#pragma unroll
    for (int tt = 0; tt < C; ++tt) {
      mac_tile(buf, tt);
#pragma unroll
      for (int u = 0; u < RW; ++u)
        wbuf[tt * RW + u] = __builtin_nontemporal_load(wtile((c + 1) * CH + tt * RW + u));
    }
    store_chunk(c + 1);
  }
  __syncthreads();
  {
    const unsigned short* buf = xb + (c & 1) * 2 * NB * P;
#pragma unroll
    for (int tt = 0; tt < C; ++tt)
      if (c * C + tt < nk) mac_tile(buf, tt);  // (wave-uniform)
  }

  // the residual epilogue's old residual and the next consumer's gain
  // (outputs idx = tid + 256 j = b * rows + r), while the waves finish
  // (an unsplit item's; a split one loads its share's in gemv_finish_coop)
  constexpr int kXold = (kRows * NB + 255) / 256;
  float x_old[kXold], xo_g[kXold];
  if (MODE == kResid && S == 1) {
#pragma unroll
    for (int j = 0; j < kXold; ++j) {
      const int idx = tid + j * 256;
      if (idx < kRows * B) {
        const size_t n = (size_t)rg * kRows + idx % kRows;
        x_old[j] = (a.res_in != nullptr ? a.res_in : a.out)[(size_t)(idx / kRows) * a.N + n];
        xo_g[j] = a.xo_hi != nullptr ? a.xo_gain[n] : 0.f;
      }
    }
  }
  mark(3);
  __syncthreads();  // every wave is done with the input buffers (s_res shares them)
#pragma unroll
  for (int u = 0; u < RW; ++u)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int col = cb * 16 + (lane & 15);
      const float sc = norm && col < B ? s_inv[col] : 1.f;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s_res[((wave + 4 * u) * 16 + (lane >> 4) * 4 + r) * NB + col] = acc[u][cb][r] * sc;
    }
  __syncthreads();
  mark(4);
  if constexpr (MODE == kStore || MODE == kResid || MODE == kSwiGLU) {
    if (S > 1) {
      gemv_finish_coop<NB, MODE, kRows>(a, rg, s, s_res, mark);
      return;
    }
  }
  gemv_finish<NB, MODE, kRows>(a, done, rg, s, kRows, s_res, s_flag, x_old, xo_g, mark);
}

// ------------------------------------------------------------------ attention

// LDS of an attention item with NW waves.  part (partial q.k sums of the
// page being scored) and acc (the waves' outputs, for the final merge) are
// never live at the same time.
template <int D, int G, int NW, int PW = 1>
struct AttnSmem {
  static constexpr int LPT = D / 8;       // lanes per token row in one 1 KB load
  static constexpr int TPI = 64 / LPT;    // tokens per load
  static constexpr int NI = kPage / TPI;  // loads per 16-token tile
  static constexpr int NV = NI * G;       // partial scores per lane per page
  static constexpr int ACC = G * 8 + 1;  // per-lane accumulators, padded against bank conflicts
  // the softmax weights of a wave's PW pages go into its partials' space
  // when that holds them, else here
  static constexpr int PX = PW > NV ? PW : 1;
  union {
    float part[NW][NV][64];
    float acc[NW][64][ACC];  // every lane's G x 8 output partials
    float ml[2][G][kMaxSplitsStaged];  // combine: (max, sum) of the splits
  };
  alignas(16) float q[G][D];
  float p[NW][PX][64];
  float m[NW][G], l[NW][G];
  float wsc[NW][G];        // per-wave rescale factors of the merge
  float mx[G], lsum[G];    // per head: overall max and sum of the item (or of all splits)
  alignas(16) unsigned short k[D];  // this step's k, v as pool elements (E4M3 codes widened)
  alignas(16) unsigned short v[D];
  unsigned flag;
};

// Pages one split of a sequence covers: every wave of an NW-wave workgroup
// holds PW pages in flight.
template <int NW, int PW>
__host__ __device__ constexpr int attn_pages_per_split() { return NW * PW; }

// The attention work of one step, held in registers by every wave: lane b
// (< B) has sequence b's position (clamped; an out-of-range one is flagged),
// its split count and its range [first, end) of item numbers.  Items are
// numbered sequence by sequence, (KV head, split) inside, so the count
// follows from the positions and no launch slot goes to an item that does
// not exist.
struct AttnList {
  int pos, nsplit, first, end;
};

template <int PPS>
__device__ inline AttnList attn_list(const AttnArgs& a) {
  const int lane = threadIdx.x & 63;
  AttnList l{0, 0, 0, 0};
  int items = 0;
  if (lane < a.B) {
    int pos = a.positions[lane];
    const int pos_lim = min(a.max_pages * kPage, a.max_pos);
    if (pos < 0 || pos >= pos_lim) {
      if (threadIdx.x == lane) set_flag(a.dev_flags, QD_DEV_BAD_POSITION);
      pos = pos < 0 ? 0 : pos_lim - 1;
    }
    const int npages = (pos + 1 + kPage - 1) / kPage;
    l.pos = pos;
    l.nsplit = (npages + PPS - 1) / PPS;
    items = a.Hkv * l.nsplit;
  }
  int inc = items;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int v = __shfl_up(inc, m);
    if (lane >= m) inc += v;
  }
  l.end = inc;
  l.first = inc - items;
  return l;
}

// Items of the step (the same in every wave).
__device__ __forceinline__ int attn_items(const AttnList& l, int B) { return __shfl(l.end, B - 1); }

// One item per (sequence b, KV head g, split s) of NW waves.  Fuses, for the
// step's token: RMSNorm of the G query heads and of the KV head over
// head_dim, NeoX RoPE at the token's position, and the bf16 append of k and
// v into the pool (by the split that owns the last page); then paged
// attention of the G query heads over the split's pages (K/V read once for
// the whole group), online softmax per wave, the waves merged in LDS, and
// for contexts longer than one split the log-sum-exp combine of the splits
// by the last split to arrive.
//
// A split covers NW*PW pages (page s*NW*PW + w + NW*j for wave w, j < PW):
// each wave issues all of its pages' K/V loads at once, before waiting for
// the q, k, v inputs.
//
// Within a wave, a 16-token page tile of K (or V) for one head is NI loads of
// 1 KB: in load i lane l holds token i*TPI + l/LPT, dims (l%LPT)*8 .. +8.
template <int D, int G, int NW, int PW, class Wait, class KV = KvBf16>
__device__ inline void attention_item(const AttnArgs& a, const AttnList& list,
                                      const float* q_gain, const float* k_gain,
                                      typename KV::Elem* pool_layer, const Done& done, int item,
                                      unsigned char* smem, const Wait& wait) {
  using Raw = typename KV::Raw;
  using SM = AttnSmem<D, G, NW, PW>;
  constexpr bool kAgent = Wait::kInLaunch;
#ifdef QD_STEP_TRACE
  auto mark = [&](int e) {
    if (a.trace != nullptr && threadIdx.x == 0) a.trace[e] = __builtin_amdgcn_s_memrealtime();
  };
#else
  auto mark = [](int) {};
#endif
  mark(0);
  constexpr int LPT = SM::LPT, TPI = SM::TPI, NI = SM::NI;
  constexpr int HALF = D / 2;
  constexpr int PPS = attn_pages_per_split<NW, PW>();
  static_assert(16 * G <= 64, "at most 4 query heads per KV head");
  SM& sm = *reinterpret_cast<SM*>(smem);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int S_max = a.S_max;
  const int Hq = a.Hq, Hkv = a.Hkv;
  // this item's sequence: the lane whose item range holds it
  const unsigned long long mine =
      __ballot(lane < a.B && item >= list.first && item < list.end);
  const int b = __ffsll((long long)mine) - 1;
  const int pos = __shfl(list.pos, b);
  const int nsplit = __shfl(list.nsplit, b);
  const int u = item - __shfl(list.first, b);
  const int g = u % Hkv, s = u / Hkv;
  const int ctx = pos + 1;

  const int npages = (ctx + kPage - 1) / kPage;
  const int* bt = a.block_tables + (size_t)b * a.max_pages;
  const size_t head_stride = (size_t)kPage * D;  // one (page, K|V, head) tile
  const int pg0 = s * PPS;
  const bool act = lane < HALF;
  constexpr int HPW = (G + 2 + NW - 1) / NW;  // q/k/v heads per wave in the prologue

  // Loads are issued in dependency order (they complete in order for the
  // wait counter): the block-table entries of the wave's pages, the inputs
  // of its q/k/v heads and their gains and the RoPE row, then the K/V pages.
  int phys[PW];
#pragma unroll
  for (int j = 0; j < PW; ++j) phys[j] = bt[min(pg0 + wave + NW * j, npages - 1)];

  // q/k/v head hh = wave + NW*u of the group: rows off..off+D of the QKV
  // projection; lane takes dims lane and lane + D/2.  The split partials
  // (up to 8) are loaded now and summed in order in the prologue.
  // (Inside the persistent kernel the projection is produced by the same
  // launch, so these loads wait for it: see load_inputs below.)
  auto head_row = [&](int hh) {
    return hh < G ? (g * G + hh) * D : hh == G ? Hq * D + g * D : (Hq + Hkv) * D + g * D;
  };
  const bool early = a.qkv_part == nullptr || a.qkv_S <= 8;
  float xp1[HPW][8], xp2[HPW][8], gn1[HPW], gn2[HPW];
  // The same 8 loads per value on every path (a materialised q|k|v row
  // repeats its one address; past 8 splits the loads go unused and
  // split_sum reads the partials later): with no branch between them and
  // the block-table loads issued before, the compiler's wait for a page id
  // does not also wait for these inputs.
  auto load_inputs = [&]() {
    const bool part = a.qkv_part != nullptr;
    const int rows = part ? a.qkv_rows : 1, S = part ? max(a.qkv_S, 1) : 1;
    const float* base = part ? a.qkv_part : a.qkv + (size_t)b * (Hq + 2 * Hkv) * D;
    const size_t stride = part ? (size_t)rows * a.B : 0;
#pragma unroll
    for (int uu = 0; uu < HPW; ++uu) {
      const int hh = min(wave + NW * uu, G + 1);
      const int off = head_row(hh);
      const int l2 = act ? lane : 0;
      const int n1 = off + l2, n2 = off + l2 + HALF;
      const float* p1 = base + (part ? ((size_t)(n1 / rows) * S * rows + n1 % rows) * a.B + b : n1);
      const float* p2 = base + (part ? ((size_t)(n2 / rows) * S * rows + n2 % rows) * a.B + b : n2);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xp1[uu][j] = ld_in<kAgent>(p1 + (size_t)min(j, S - 1) * stride);
        xp2[uu][j] = ld_in<kAgent>(p2 + (size_t)min(j, S - 1) * stride);
      }
    }
  };
  if constexpr (!kAgent) load_inputs();  // written by an earlier launch
#pragma unroll
  for (int uu = 0; uu < HPW; ++uu) {
    const int hh = min(wave + NW * uu, G + 1);
    const float* gain = hh < G ? q_gain : k_gain;
    const int l2 = act ? lane : 0;
    gn1[uu] = gain[l2];
    gn2[uu] = gain[l2 + HALF];
  }
  const float cs1 = a.rope_cos[(size_t)pos * HALF + (act ? lane : 0)];
  const float sn1 = a.rope_sin[(size_t)pos * HALF + (act ? lane : 0)];

  // --- the cached K/V pages of this wave (they do not depend on this
  // step's projections, so they go out before the wait).  Every load is
  // issued unconditionally: a page past the context repeats the last page
  // (its scores are masked), so no wait is forced between pages.
  Raw kr[PW][NI], vr[PW][NI];
  const Raw zero4 = KV::zero();
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    const int pg = pg0 + wave + NW * j;
    int ph = phys[j];
    if (ph < 0 || ph >= a.num_pages) {
      if (lane == 0 && pg < npages) set_flag(a.dev_flags, QD_DEV_BAD_PAGE);
      ph = 0;
    }
    const typename KV::Elem* kp = pool_layer + (((size_t)ph * 2 + 0) * Hkv + g) * head_stride;
    const typename KV::Elem* vp = pool_layer + (((size_t)ph * 2 + 1) * Hkv + g) * head_stride;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      kr[j][i] = KV::load_nt(kp + (size_t)(i * 64 + lane) * 8);
      vr[j][i] = KV::load_nt(vp + (size_t)(i * 64 + lane) * 8);
    }
  }

  wait();
  __syncthreads();  // LDS of the previous item is free
  mark(1);
  if constexpr (kAgent) load_inputs();  // written in this launch: after the wait

  // --- q/k RMSNorm + RoPE, v to bf16 (wave w takes heads w, w+NW, ...)
#pragma unroll
  for (int uu = 0; uu < HPW; ++uu) {
    const int hh = wave + NW * uu;
    if (hh >= G + 2) break;  // wave-uniform
    float x1 = 0.f, x2 = 0.f;
    if (a.qkv_part == nullptr) {
      x1 = xp1[uu][0];
      x2 = xp2[uu][0];
    } else if (early) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < a.qkv_S) { x1 += xp1[uu][j]; x2 += xp2[uu][j]; }
    } else {
      const int off = head_row(hh), l2 = act ? lane : 0;
      x1 = split_sum<kAgent>(a.qkv_part, a.qkv_S, a.B, a.qkv_rows, off + l2, b);
      x2 = split_sum<kAgent>(a.qkv_part, a.qkv_S, a.B, a.qkv_rows, off + l2 + HALF, b);
    }
    if (!act) { x1 = 0.f; x2 = 0.f; }
    if (hh <= G) {  // q heads and k: RMSNorm over head_dim, gain, RoPE
      const float ss = wave_sum(x1 * x1 + x2 * x2);
      const float inv = rsqrtf(ss / (float)D + a.eps);
      if (act) {
        const float y1 = x1 * inv * gn1[uu], y2 = x2 * inv * gn2[uu];
        const float r1 = y1 * cs1 - y2 * sn1, r2 = y2 * cs1 + y1 * sn1;
        if (hh < G) {
          sm.q[hh][lane] = r1 * a.scale;
          sm.q[hh][lane + HALF] = r2 * a.scale;
          if (a.tap_q != nullptr && s == 0) {
            float* tq = a.tap_q + ((size_t)b * Hq + g * G + hh) * D;
            tq[lane] = r1; tq[lane + HALF] = r2;
          }
        } else {
          sm.k[lane] = KV::encode(r1, a.k_inv);
          sm.k[lane + HALF] = KV::encode(r2, a.k_inv);
          if (a.tap_k != nullptr && s == 0) {
            float* tk = a.tap_k + ((size_t)b * Hkv + g) * D;
            tk[lane] = r1; tk[lane + HALF] = r2;
          }
        }
      }
    } else if (act) {
      sm.v[lane] = KV::encode(x1, a.v_inv);
      sm.v[lane + HALF] = KV::encode(x2, a.v_inv);
    }
  }
  __syncthreads();

  // --- append k, v of this step (the split owning the last page does it).
  // A prefill chunk's rows attend to one another's K/V, so its layer runs
  // two launches: the first only appends, the second only attends (its own
  // k, v come from LDS, the same bits the first launch wrote).
  const int kv_mode = kAgent ? kAppendAttend : a.kv_mode;
  if (kv_mode != kAttendOnly && s == nsplit - 1) {
    const int page = bt[pos / kPage];
    if (page < 0 || page >= a.num_pages) {
      if (tid == 0) set_flag(a.dev_flags, QD_DEV_BAD_PAGE);
    } else {
      typename KV::Elem* kd = pool_layer + (((size_t)page * 2 + 0) * Hkv + g) * head_stride +
                              (size_t)(pos % kPage) * D;
      typename KV::Elem* vd = pool_layer + (((size_t)page * 2 + 1) * Hkv + g) * head_stride +
                              (size_t)(pos % kPage) * D;
      for (int i = tid; i < D; i += NW * 64) {
        kd[i] = (typename KV::Elem)sm.k[i];
        vd[i] = (typename KV::Elem)sm.v[i];
      }
    }
  }
  if (kv_mode == kAppendOnly) return;  // uniform over the workgroup

  mark(2);
  // --- paged attention over this wave's pages
  const int dch = lane % LPT;
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // softmax state of head (lane % G)
  const Raw kcur = KV::from_slots(&sm.k[dch * 8]);
  const Raw vcur = KV::from_slots(&sm.v[dch * 8]);

  // The wave's PW pages are scored first, then one online-softmax update
  // covers all of them (one max and one sum across the lanes instead of one
  // per page), then the values.  Pages past the context were loaded, not
  // used (wave-uniform).
  float sc[PW];  // lane u < 16G: score of (token u/G, head u%G) of page j
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    const int pg = pg0 + wave + NW * j;
    sc[j] = -INFINITY;
    if (pg >= npages) continue;
    // partial q.k over this lane's 8 dims, for its NI tokens and G heads
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = pg * kPage + i * TPI + lane / LPT;
      Raw kk = kr[j][i];
      if (tok == pos) { kk = kcur; vr[j][i] = vcur; }
      if (tok >= ctx) { kk = zero4; vr[j][i] = zero4; }
      float kf[8];
      KV::unpack(kk, kf, a.k_scale);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const f32x4 q0 = *reinterpret_cast<const f32x4*>(&sm.q[h][dch * 8]);
        const f32x4 q1 = *reinterpret_cast<const f32x4*>(&sm.q[h][dch * 8 + 4]);
        float p = 0.f;
        p = fmaf(q0.x, kf[0], p); p = fmaf(q0.y, kf[1], p);
        p = fmaf(q0.z, kf[2], p); p = fmaf(q0.w, kf[3], p);
        p = fmaf(q1.x, kf[4], p); p = fmaf(q1.y, kf[5], p);
        p = fmaf(q1.z, kf[6], p); p = fmaf(q1.w, kf[7], p);
        sm.part[wave][i * G + h][lane] = p;
      }
    }
    __builtin_amdgcn_wave_barrier();
    // lane u < 16G owns score (token u/G, head u%G): sum the LPT partials
    // (the wave's LDS operations run in order, so the next page's partials
    // are written after these reads)
    if (lane < 16 * G) {
      const int t = lane / G, h = lane % G;
      const float* src = &sm.part[wave][(t / TPI) * G + h][(t % TPI) * LPT];
      float sum = 0.f;
#pragma unroll
      for (int jj = 0; jj < LPT; jj += 4) {
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(src + jj);
        sum += v4.x; sum += v4.y; sum += v4.z; sum += v4.w;
      }
      if (pg * kPage + t < ctx) sc[j] = sum;
    }
  }
  float mx = sc[0];
#pragma unroll
  for (int j = 1; j < PW; ++j) mx = fmaxf(mx, sc[j]);
#pragma unroll
  for (int m = G; m < 64; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
  const float m_new = fmaxf(m_run, mx);
  float pj[PW], psum = 0.f;
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    pj[j] = (sc[j] == -INFINITY) ? 0.f : expf(sc[j] - m_new);
    psum += pj[j];
  }
  const float alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
#pragma unroll
  for (int m = G; m < 64; m <<= 1) psum += __shfl_xor(psum, m);
  l_run = l_run * alpha + psum;
  m_run = m_new;
  // the weights of every page, in the partials' space (free now) if it holds them
  float* const pw = PW <= SM::NV ? &sm.part[wave][0][0] : &sm.p[wave][0][0];
#pragma unroll
  for (int j = 0; j < PW; ++j) pw[j * 64 + lane] = pj[j];
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float al = __shfl(alpha, h);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] *= al;
  }
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    if (pg0 + wave + NW * j >= npages) break;  // wave-uniform
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = i * TPI + lane / LPT;
      float vf[8];
      KV::unpack(vr[j][i], vf, a.v_scale);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pv = pw[j * 64 + t * G + h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv, vf[e], acc[h][e]);
      }
    }
  }
  __builtin_amdgcn_wave_barrier();

  mark(3);
  // --- merge the waves (and the TPI token groups inside each) through LDS:
  // every lane stores its partials, one thread per (wave, head) the factor
  // exp(m_w - M), then each output sums its NW * TPI partials
  __syncthreads();  // every wave is done with part (acc aliases it)
  if (lane < G) { sm.m[wave][lane] = m_run; sm.l[wave][lane] = l_run; }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) sm.acc[wave][lane][h * 8 + e] = acc[h][e];
  __syncthreads();
  if (tid < NW * G) {
    const int w = tid / G, h = tid % G;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, sm.m[w2][h]);
    const float mw = sm.m[w][h];
    sm.wsc[w][h] = mw == -INFINITY ? 0.f : expf(mw - M);
    if (w == 0) sm.mx[h] = M;
  }
  __syncthreads();
  if (tid < G) {
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) L += sm.l[w][tid] * sm.wsc[w][tid];
    sm.lsum[tid] = L;
  }
  __syncthreads();

  const size_t qh0 = (size_t)b * Hq + (size_t)g * G;  // first query head row of this group
  for (int idx = tid; idx < G * D; idx += NW * 64) {
    const int h = idx / D, d = idx % D;
    const int dc = d / 8, e = d % 8;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      float ow = 0.f;
#pragma unroll
      for (int grp = 0; grp < TPI; ++grp) ow += sm.acc[w][grp * LPT + dc][h * 8 + e];
      o += ow * sm.wsc[w][h];
    }
    const float M = sm.mx[h], L = sm.lsum[h];
    if (nsplit == 1) {
      st_agent(a.out + (qh0 + h) * D + d, o / L);
      if (a.out_hi != nullptr) split_hilo(o / L, a.out_hi, a.out_lo, (qh0 + h) * D + d);
    } else {
      st_agent(a.o_part + ((qh0 + h) * S_max + s) * D + d, o);
      if (d == 0) {
        st_agent(a.ml_part + ((qh0 + h) * S_max + s) * 2 + 0, M);
        st_agent(a.ml_part + ((qh0 + h) * S_max + s) * 2 + 1, L);
      }
    }
  }
  if (nsplit == 1) {
    mark(4);
    signal_done(done);
    mark(7);
    return;
  }

  unsigned* cnt = &a.counters[((size_t)b * Hkv + g) * kCntStride];
  mark(4);
  if (!arrive_last(cnt, (unsigned)nsplit, &sm.flag)) return;
  mark(5);
  // (max, sum) of every split into LDS, and (for up to kFastSplits splits) each
  // 4-output chunk's split partials into registers with one 16-byte
  // device-scope load per split, in the same round trip; then per head the
  // overall max and the splits' factors exp(m_s - M)
  constexpr int kChunks = G * D / 4;  // 4-float output chunks, one per thread
  static_assert(kChunks <= NW * 64, "one chunk per thread");
  constexpr int kFastSplits = 24;  // (8K context at batch 1: 22 splits)
  f32x4 ov[kFastSplits];
  if (nsplit <= kFastSplits && tid < kChunks) {
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        a.o_part, 0, (int)((size_t)a.B * Hq * S_max * D * 4), kBufferWord3);
    const int base = (int)(((qh0 + (4 * tid) / D) * S_max) * D + (4 * tid) % D) * 4;
#pragma unroll
    for (int j = 0; j < kFastSplits; ++j)
      if (j < nsplit)
        ov[j] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, base + j * D * 4, 0, kDeviceScope));
  }
  for (int i = tid; i < G * nsplit; i += NW * 64) {
    const int h = i / nsplit, s2 = i % nsplit;
    const float* ml = a.ml_part + ((qh0 + h) * S_max + s2) * 2;
    sm.ml[0][h][s2] = ld_agent(ml);
    sm.ml[1][h][s2] = ld_agent(ml + 1);
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int s2 = 0; s2 < nsplit; ++s2) M = fmaxf(M, sm.ml[0][tid][s2]);
    float L = 0.f;
    for (int s2 = 0; s2 < nsplit; ++s2) {
      const float f = expf(sm.ml[0][tid][s2] - M);
      sm.ml[0][tid][s2] = f;
      L += sm.ml[1][tid][s2] * f;
    }
    sm.lsum[tid] = L;
  }
  __syncthreads();
  if (nsplit <= kFastSplits) {
    if (tid < kChunks) {
      const int h = (4 * tid) / D, d0 = (4 * tid) % D;
      f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kFastSplits; ++j)
        if (j < nsplit) o += ov[j] * sm.ml[0][h][j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float r = o[e] / sm.lsum[h];
        st_agent(a.out + (qh0 + h) * D + d0 + e, r);
        if (a.out_hi != nullptr) split_hilo(r, a.out_hi, a.out_lo, (qh0 + h) * D + d0 + e);
      }
    }
  } else {
    constexpr int kOut = (G * D + NW * 64 - 1) / (NW * 64);  // outputs per thread
#pragma unroll
    for (int k = 0; k < kOut; ++k) {
      const int idx = tid + k * NW * 64;
      if (idx >= G * D) break;
      const int h = idx / D, d = idx % D;
      float o = 0.f;
      const float* op = a.o_part + (qh0 + h) * S_max * D + d;
      for (int s0 = 0; s0 < nsplit; s0 += 16) {
        float w16[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) w16[j] = ld_agent(op + (size_t)min(s0 + j, nsplit - 1) * D);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (s0 + j < nsplit) o += w16[j] * sm.ml[0][h][s0 + j];
      }
      const float r = o / sm.lsum[h];
      st_agent(a.out + (qh0 + h) * D + d, r);
      if (a.out_hi != nullptr) split_hilo(r, a.out_hi, a.out_lo, (qh0 + h) * D + d);
    }
  }
  if (tid == 0) reset_counter(cnt);
  mark(6);
  signal_done(done);
  mark(7);
}

// ------------------------------------------------------------------ streaming step

// Waits (thread 0 polls, the workgroup then proceeds together) until this
// workgroup's flag reaches `phase` (see signal_done).  Bounded: after
// `limit` polls it records QD_DEV_TIMEOUT and sets the abort flag, after
// which every later wait falls through, so every workgroup always reaches
// the end of the kernel.
struct Waiter {
  static constexpr bool kInLaunch = true;
  const unsigned* flag;
  unsigned phase;
  unsigned* abort_flag;
  int* dev_flags;
  unsigned limit;
  __device__ void operator()() const {
    if (threadIdx.x == 0) {
      unsigned n = 0;
      while (ld_agent(flag) < phase) {
        if ((n & 63) == 0 && ld_agent(abort_flag) != 0u) break;
        if (++n > limit) {
          set_flag(dev_flags, QD_DEV_TIMEOUT);
          st_agent(abort_flag, 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
  }
};

}  // namespace qd
