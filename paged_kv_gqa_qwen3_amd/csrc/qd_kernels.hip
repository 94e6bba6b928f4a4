// HIP kernels of the decode step, written for CDNA4 (gfx950, wave64).
//
// Decode is memory bound: a step streams every weight once (the pages find
// bf16 GEMV to be the dominant cost of decode, "GPU 算子与执行优化", Part 2
// kernel table), so the kernels are organised around one rule: keep enough
// 16-byte loads in flight to saturate HBM, and do everything else (norms,
// RoPE, KV append, residual adds, SwiGLU, argmax) in the prologue or epilogue
// of the kernel that already has the data on chip.
#include <hip/hip_runtime.h>

#include <math.h>

#include "qd.h"
#include "qd_internal.h"

namespace qd {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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

__device__ __forceinline__ void unpack8(const u32x4& w, float* f) {
  f[0] = bf_lo(w.x); f[1] = bf_hi(w.x); f[2] = bf_lo(w.y); f[3] = bf_hi(w.y);
  f[4] = bf_lo(w.z); f[5] = bf_hi(w.z); f[6] = bf_lo(w.w); f[7] = bf_hi(w.w);
}

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

// Cross-workgroup hand-off of partial results ("last workgroup finishes").
//
// Partials and counters are written and read with agent-scope relaxed atomic
// accesses (coherent across the XCDs' L2s on gfx950).  The arriving
// workgroup waits until all of its partial stores are acknowledged before it
// increments the counter, and the last arrival reads the partials with
// agent-scope loads.  Plain __threadfence() would order the same way but costs
// an L2 writeback and invalidate per wave, measured at ~0.2 us of serialised
// device time per workgroup on MI355X.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_agent(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns true in the workgroup that arrives last at `counter`.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected,
                                            unsigned* s_flag) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's agent-scope stores are performed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (prev == expected - 1) ? 1u : 0u;
  }
  __syncthreads();
  return *s_flag != 0;
}

// sum_{s < n} p[s * stride] in increasing s, with the loads issued 8 at a
// time (unconditional, clamped index) so that they overlap.
__device__ __forceinline__ float sum_strided(const float* p, int n, size_t stride) {
  float sum = 0.f;
  for (int s0 = 0; s0 < n; s0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ld_agent(p + (size_t)min(s0 + j, n - 1) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < n) sum += v[j];
  }
  return sum;
}

__device__ __forceinline__ void reset_counter(unsigned* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ repack

// Row-major [rows][K] bf16 -> tile-major (see qd_internal.h).  Source row
// tile j lands in destination row tile j * tile_mul + tile_add, which fuses
// q|k|v (tile_add = row offset / 16) and pairs gate|up (tile_mul = 2).
__global__ void repack_kernel(const uint16_t* __restrict__ src, int rows, int K,
                              uint16_t* __restrict__ dst, int tile_mul, int tile_add) {
  const int KT = K / kTileCols;
  const size_t n = (size_t)(rows / kTileRows) * KT * 64;
  for (size_t c = blockIdx.x * (size_t)blockDim.x + threadIdx.x; c < n;
       c += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(c % 64);
    const size_t t = c / 64;
    const int kt = (int)(t % KT);
    const int rt = (int)(t / KT);
    const uint16_t* s = src + (size_t)(rt * kTileRows + lane % 16) * K + kt * kTileCols +
                        (lane / 16) * 8;
    const size_t drt = (size_t)rt * tile_mul + tile_add;
    uint16_t* d = dst + (drt * KT + kt) * kTileElems + lane * 8;
    *reinterpret_cast<u32x4*>(d) = *reinterpret_cast<const u32x4*>(s);
  }
}

__global__ void bf16_to_f32_kernel(const uint16_t* __restrict__ src, float* __restrict__ dst,
                                   int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = __uint_as_float((unsigned)src[i] << 16);
}

// ------------------------------------------------------------------ embedding

// x[b] = E[token_b] (exact bf16 -> fp32), read from the packed table, plus
// the sums of squares of x over each group of 64 columns (the RMSNorm of the
// first QKV projection consumes them).
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
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
    a.x[(size_t)b * a.H + k] = xv;
    const float ss = wave_sum(xv * xv);
    if (lane == 0) a.ssq_out[(size_t)(base / 64) * a.Bmax + b] = ss;
  }
}

// out[b][k] = x[b][k] * rsqrt(sum(ssq partials)/H + eps) * gain[k]
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const float* x, const float* ssq,
                                                           const float* gain, int H, int Bmax,
                                                           float eps, float* out) {
  const int b = blockIdx.x;
  __shared__ float s_inv;
  if (threadIdx.x == 0) {
    float ss = 0.f;
    for (int g = 0; g < H / 64; ++g) ss += ssq[(size_t)g * Bmax + b];
    s_inv = rsqrtf(ss / (float)H + eps);
  }
  __syncthreads();
  for (int k = threadIdx.x; k < H; k += blockDim.x)
    out[(size_t)b * H + k] = x[(size_t)b * H + k] * s_inv * gain[k];
}

// ------------------------------------------------------------------ GEMV

// y[b][n] = sum_k W[n][k] h[b][k], h = x or RMSNorm(x), W packed bf16.
//
// Workgroup = 4 waves = 64 output rows (one 16-row tile per wave) x one K
// slice of kps tiles.  Each wave streams its slice of weight tiles with one
// 16-byte load per lane per 1 KB tile, up to CH tiles in flight.  The K
// slice of the (normalised) input sits in LDS.
//   NB <= 4 : VALU path, fp32 input, NB batch columns, fp32 FMA.
//   NB >= 16: MFMA path, NB/16 blocks of 16 batch columns,
//             v_mfma_f32_16x16x32_bf16 with the weight tile as operand A and
//             the input as a pair of bf16 (hi = bf16(x), lo = bf16(x - hi)),
//             two MFMAs per tile: ~16 significant bits of input instead of 8
//             (bf16 inputs alone move a 36-layer model's logits by ~2% of
//             their maximum, beyond the step's 2e-2 tolerance).
// With S > 1 splits of K, each workgroup writes its partial tile and the last
// to arrive sums the S partials in split order (deterministic) and runs the
// epilogue.
template <int NB, int MODE>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  constexpr bool kMfma = NB >= 16;
  constexpr int NCB = kMfma ? NB / 16 : 1;
  constexpr int CH = 20;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float s_inv[kMaxBatch];
  __shared__ float s_res[kRowsPerGroup * NB];
  __shared__ unsigned s_flag;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int B = a.B, S = a.S;
  const int rg = blockIdx.x / S, s = blockIdx.x - rg * S;
  const int KT = a.K / kTileCols;
  const int kt0 = s * a.kps;
  const int kt1 = min(KT, kt0 + a.kps);
  const int nk = kt1 - kt0;
  const int Ks = nk * kTileCols;
  const int rt = rg * 4 + wave;
  const u32x4* wp = reinterpret_cast<const u32x4*>(a.w) + ((size_t)rt * KT + kt0) * 64 + lane;

  // First chunk of weight loads goes out before the input is staged.  Every
  // load is issued unconditionally (tile index clamped to the slice) so that
  // the loads stay in flight together; only the compute is guarded.
  u32x4 wbuf[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i)
    wbuf[i] = __builtin_nontemporal_load(wp + (size_t)min(i, nk - 1) * 64);

  // RMSNorm scale per batch column from the producer's partial sums of
  // squares: wave w reduces columns w, w+4, ... over its lanes (fixed order).
  if (a.ssq != nullptr) {
    const int ng = a.K / 64;
    for (int b = wave; b < B; b += 4) {
      float ss = 0.f;
      for (int g0 = 0; g0 < ng; g0 += 64) {
        const int g = g0 + lane;
        ss += g < ng ? a.ssq[(size_t)g * a.Bmax + b] : 0.f;
      }
      ss = wave_sum(ss);
      if (lane == 0) s_inv[b] = rsqrtf(ss / (float)a.K + a.eps);
    }
    __syncthreads();
  }

  // Stage the input slice: fp32 [NB][Ks] (VALU), or bf16 hi [NB][Ks + 8]
  // followed by bf16 lo [NB][Ks + 8] (MFMA).
  const int P = kMfma ? Ks + 8 : Ks;
  {
    const int total = NB * Ks;
    for (int idx = tid; idx < total; idx += 256) {
      const int b = idx / Ks, k = idx - b * Ks;
      float v = 0.f;
      if (b < B) {
        const int kk = kt0 * kTileCols + k;
        v = a.x[(size_t)b * a.K + kk];
        if (a.ssq != nullptr) v = v * s_inv[b] * a.gain[kk];
      }
      if (kMfma) {
        unsigned short* xs = reinterpret_cast<unsigned short*>(smem);
        const unsigned short hi = f2bf(v);
        xs[b * P + k] = hi;
        xs[NB * P + b * P + k] = f2bf(v - __uint_as_float((unsigned)hi << 16));
      } else {
        reinterpret_cast<float*>(smem)[b * P + k] = v;
      }
    }
  }
  __syncthreads();

  float acc_v[kMfma ? 1 : NB];
  f32x4 acc_m[NCB];
#pragma unroll
  for (int b = 0; b < (kMfma ? 1 : NB); ++b) acc_v[b] = 0.f;
#pragma unroll
  for (int c = 0; c < NCB; ++c) acc_m[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < nk; c0 += CH) {
    const int n = min(CH, nk - c0);
    if (c0 > 0) {
#pragma unroll
      for (int i = 0; i < CH; ++i)
        wbuf[i] = __builtin_nontemporal_load(wp + (size_t)min(c0 + i, nk - 1) * 64);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (i < n) {
        const int t = c0 + i;
        if constexpr (kMfma) {
          const unsigned short* xs = reinterpret_cast<const unsigned short*>(smem);
          const bf16x8 wa = __builtin_bit_cast(bf16x8, wbuf[i]);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const int off = (cb * 16 + (lane & 15)) * P + t * kTileCols + (lane >> 4) * 8;
            const u32x4 xh = *reinterpret_cast<const u32x4*>(xs + off);
            const u32x4 xl = *reinterpret_cast<const u32x4*>(xs + NB * P + off);
            acc_m[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                wa, __builtin_bit_cast(bf16x8, xh), acc_m[cb], 0, 0, 0);
            acc_m[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                wa, __builtin_bit_cast(bf16x8, xl), acc_m[cb], 0, 0, 0);
          }
        } else {
          const float* xs = reinterpret_cast<const float*>(smem) + t * kTileCols + (lane >> 4) * 8;
          float wf[8];
          unpack8(wbuf[i], wf);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(xs + b * P);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(xs + b * P + 4);
            float acc = acc_v[b];
            acc = fmaf(wf[0], x0.x, acc); acc = fmaf(wf[1], x0.y, acc);
            acc = fmaf(wf[2], x0.z, acc); acc = fmaf(wf[3], x0.w, acc);
            acc = fmaf(wf[4], x1.x, acc); acc = fmaf(wf[5], x1.y, acc);
            acc = fmaf(wf[6], x1.z, acc); acc = fmaf(wf[7], x1.w, acc);
            acc_v[b] = acc;
          }
        }
      }
    }
  }

  // Row results of this workgroup -> s_res[64 rows][NB].
  if constexpr (kMfma) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s_res[(wave * 16 + (lane >> 4) * 4 + r) * NB + cb * 16 + (lane & 15)] = acc_m[cb][r];
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v = acc_v[b];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane < 16) s_res[(wave * 16 + lane) * NB + b] = v;
    }
  }
  __syncthreads();

  const int rows = kRowsPerGroup;
  if (S > 1) {
    float* mine = a.part + (size_t)(rg * S + s) * rows * B;
    for (int idx = tid; idx < rows * B; idx += 256) {
      const int r = idx / B, b = idx - r * B;
      st_agent(mine + idx, s_res[r * NB + b]);
    }
    if (!arrive_last(&a.counters[rg], (unsigned)S, &s_flag)) return;
    const float* all = a.part + (size_t)rg * S * rows * B;
    for (int idx = tid; idx < rows * B; idx += 256) {
      const float sum = sum_strided(all + idx, S, (size_t)rows * B);
      const int r = idx / B, b = idx - r * B;
      s_res[r * NB + b] = sum;
    }
    if (tid == 0) reset_counter(&a.counters[rg]);
    __syncthreads();
  }

  const int N = a.N;
  const size_t row0 = (size_t)rg * rows;
  if constexpr (MODE == kStore) {
    for (int idx = tid; idx < rows * B; idx += 256) {
      const int b = idx / rows, r = idx - b * rows;
      a.out[(size_t)b * N + row0 + r] = s_res[r * NB + b];
    }
  } else if constexpr (MODE == kResid) {
    for (int base = wave * 64; base < rows * B; base += 256) {
      const int b = base / rows, r = lane;
      float* px = a.out + (size_t)b * N + row0 + r;
      const float xv = *px + s_res[r * NB + b];
      *px = xv;
      const float ss = wave_sum(xv * xv);
      if (lane == 0) a.ssq_out[(size_t)rg * a.Bmax + b] = ss;
    }
  } else if constexpr (MODE == kSwiGLU) {
    // rows of this group: [gate j][up j][gate j+1][up j+1], 16 each
    const int half = N / 2;
    for (int idx = tid; idx < 32 * B; idx += 256) {
      const int b = idx / 32, c = idx - b * 32;
      const int q2 = c / 16, i = c % 16;
      const float gv = s_res[(q2 * 32 + i) * NB + b];
      const float uv = s_res[(q2 * 32 + 16 + i) * NB + b];
      const float sv = gv / (1.f + expf(-gv));
      a.out[(size_t)b * half + (size_t)rg * 32 + c] = sv * uv;
    }
  } else {  // kArgmax
    if (a.logits != nullptr) {
      for (int idx = tid; idx < rows * B; idx += 256) {
        const int b = idx / rows, r = idx - b * rows;
        a.logits[(size_t)b * N + row0 + r] = s_res[r * NB + b];
      }
    }
    for (int b = wave; b < B; b += 4) {
      float bv = s_res[lane * NB + b];
      int bi = (int)row0 + lane;
      wave_amax(bv, bi);
      if (lane == 0) {
        st_agent(a.amax_val + (size_t)rg * a.Bmax + b, bv);
        st_agent(a.amax_idx + (size_t)rg * a.Bmax + b, bi);
      }
    }
    const int NRG = N / rows;
    if (!arrive_last(a.amax_counter, (unsigned)NRG, &s_flag)) return;
    for (int b = wave; b < B; b += 4) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int g = lane; g < NRG; g += 64)
        amax_merge(bv, bi, ld_agent(a.amax_val + (size_t)g * a.Bmax + b),
                   ld_agent(a.amax_idx + (size_t)g * a.Bmax + b));
      wave_amax(bv, bi);
      if (lane == 0) a.next_ids[b] = bi == 0x7fffffff ? -1 : bi;
    }
    if (tid == 0) reset_counter(a.amax_counter);
  }
}

// ------------------------------------------------------------------ attention

// One workgroup per (sequence b, KV head g, split s).  Fuses, for the step's
// token: RMSNorm of the G query heads and of the KV head over head_dim, NeoX
// RoPE at the token's position, and the bf16 append of k and v into the pool
// (by the split that owns the last page); then paged attention of the G
// query heads over the split's pages (K/V read once for the whole group),
// online softmax, and the log-sum-exp combine of the splits by the last
// workgroup to arrive.  The split count is derived on the device from the
// position, so one launch shape (and one captured graph) serves every context.
//
// Within a wave, a 16-token page tile of K (or V) for one head is NI loads of
// 1 KB: in load i lane l holds token i*TPI + l/LPT, dims (l%LPT)*8 .. +8.
template <int D, int G>
__global__ __launch_bounds__(256) void attention_kernel(AttnArgs a) {
  constexpr int LPT = D / 8;
  constexpr int TPI = 64 / LPT;
  constexpr int NI = kPage / TPI;
  constexpr int NV = NI * G;
  constexpr int HALF = D / 2;
  static_assert(16 * G <= 64, "at most 4 query heads per KV head");
  __shared__ float s_q[G][D];
  __shared__ __align__(16) unsigned short s_k[D];
  __shared__ __align__(16) unsigned short s_v[D];
  __shared__ __align__(16) float s_part[4][NV][64];
  __shared__ float s_p[4][64];
  __shared__ float s_acc[4][G * 8][64];
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ unsigned s_flag;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int S_max = a.S_max;
  const int s = blockIdx.x % S_max;
  const int bg = blockIdx.x / S_max;
  const int g = bg % a.Hkv, b = bg / a.Hkv;

  int pos = a.positions[b];
  const int pos_lim = min(a.max_pages * kPage, a.max_pos);
  if (pos < 0 || pos >= pos_lim) {
    if (tid == 0 && s == 0 && g == 0) set_flag(a.dev_flags, QD_DEV_BAD_POSITION);
    pos = pos < 0 ? 0 : pos_lim - 1;
  }
  const int ctx = pos + 1;
  const int npages = (ctx + kPage - 1) / kPage;
  int pps = (npages + S_max - 1) / S_max;
  if (pps < kMinPagesPerSplit) pps = kMinPagesPerSplit;
  const int nsplit = (npages + pps - 1) / pps;
  if (s >= nsplit) return;
  const int pg0 = s * pps, pg1 = min(npages, pg0 + pps);
  const int* bt = a.block_tables + (size_t)b * a.max_pages;
  const int Hq = a.Hq, Hkv = a.Hkv;
  const float* row = a.qkv + (size_t)b * (Hq + 2 * Hkv) * D;

  // --- q/k RMSNorm + RoPE, v to bf16 (wave w takes heads w, w+4, ...)
  for (int hh = wave; hh < G + 2; hh += 4) {
    const float* src;
    const float* gain = nullptr;
    if (hh < G) {
      src = row + (size_t)(g * G + hh) * D;
      gain = a.q_gain;
    } else if (hh == G) {
      src = row + (size_t)Hq * D + (size_t)g * D;
      gain = a.k_gain;
    } else {
      src = row + (size_t)(Hq + Hkv) * D + (size_t)g * D;
    }
    const bool act = lane < HALF;
    float x1 = 0.f, x2 = 0.f;
    if (act) { x1 = src[lane]; x2 = src[lane + HALF]; }
    if (gain != nullptr) {
      const float ss = wave_sum(x1 * x1 + x2 * x2);
      const float inv = rsqrtf(ss / (float)D + a.eps);
      if (act) {
        const float y1 = x1 * inv * gain[lane], y2 = x2 * inv * gain[lane + HALF];
        const float c = a.rope_cos[(size_t)pos * HALF + lane];
        const float sn = a.rope_sin[(size_t)pos * HALF + lane];
        const float r1 = y1 * c - y2 * sn, r2 = y2 * c + y1 * sn;
        if (hh < G) {
          s_q[hh][lane] = r1 * a.scale;
          s_q[hh][lane + HALF] = r2 * a.scale;
          if (a.tap_q != nullptr && s == 0) {
            float* tq = a.tap_q + ((size_t)b * Hq + g * G + hh) * D;
            tq[lane] = r1; tq[lane + HALF] = r2;
          }
        } else {
          s_k[lane] = f2bf(r1);
          s_k[lane + HALF] = f2bf(r2);
          if (a.tap_k != nullptr && s == 0) {
            float* tk = a.tap_k + ((size_t)b * Hkv + g) * D;
            tk[lane] = r1; tk[lane + HALF] = r2;
          }
        }
      }
    } else if (act) {
      s_v[lane] = f2bf(x1);
      s_v[lane + HALF] = f2bf(x2);
    }
  }
  __syncthreads();

  // --- append k, v of this step (the split owning the last page does it)
  const size_t head_stride = (size_t)kPage * D;  // one (page, K|V, head) tile
  if (s == nsplit - 1) {
    const int page = bt[pos / kPage];
    if (page < 0 || page >= a.num_pages) {
      if (tid == 0) set_flag(a.dev_flags, QD_DEV_BAD_PAGE);
    } else {
      uint16_t* kd = a.pool_layer + (((size_t)page * 2 + 0) * Hkv + g) * head_stride +
                     (size_t)(pos % kPage) * D;
      uint16_t* vd = a.pool_layer + (((size_t)page * 2 + 1) * Hkv + g) * head_stride +
                     (size_t)(pos % kPage) * D;
      for (int i = tid; i < D; i += 256) { kd[i] = s_k[i]; vd[i] = s_v[i]; }
    }
  }

  // --- paged attention over this split's pages, page pg0+wave, +4, ...
  const int dch = lane % LPT;
  float qreg[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) qreg[h][e] = s_q[h][dch * 8 + e];
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // softmax state of head (lane % G)
  const u32x4 kcur = *reinterpret_cast<const u32x4*>(&s_k[dch * 8]);
  const u32x4 vcur = *reinterpret_cast<const u32x4*>(&s_v[dch * 8]);
  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};

  for (int pg = pg0 + wave; pg < pg1; pg += 4) {
    int phys = bt[pg];
    if (phys < 0 || phys >= a.num_pages) {
      if (lane == 0) set_flag(a.dev_flags, QD_DEV_BAD_PAGE);
      phys = 0;
    }
    const u32x4* kp = reinterpret_cast<const u32x4*>(
        a.pool_layer + (((size_t)phys * 2 + 0) * Hkv + g) * head_stride);
    const u32x4* vp = reinterpret_cast<const u32x4*>(
        a.pool_layer + (((size_t)phys * 2 + 1) * Hkv + g) * head_stride);
    u32x4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      kr[i] = __builtin_nontemporal_load(kp + i * 64 + lane);
      vr[i] = __builtin_nontemporal_load(vp + i * 64 + lane);
    }
    // partial q.k over this lane's 8 dims, for its NI tokens and G heads
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = pg * kPage + i * TPI + lane / LPT;
      if (tok == pos) { kr[i] = kcur; vr[i] = vcur; }
      if (tok >= ctx) { kr[i] = zero4; vr[i] = zero4; }
      float kf[8];
      unpack8(kr[i], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) p = fmaf(qreg[h][e], kf[e], p);
        s_part[wave][i * G + h][lane] = p;
      }
    }
    __builtin_amdgcn_wave_barrier();
    // lane u < 16G owns score (token u/G, head u%G): sum the LPT partials
    float sc = -INFINITY;
    if (lane < 16 * G) {
      const int t = lane / G, h = lane % G;
      const float* src = &s_part[wave][(t / TPI) * G + h][(t % TPI) * LPT];
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < LPT; j += 4) {
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(src + j);
        sum += v4.x; sum += v4.y; sum += v4.z; sum += v4.w;
      }
      if (pg * kPage + t < ctx) sc = sum;
    }
    float mx = sc;
#pragma unroll
    for (int m = G; m < 64; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    const float m_new = fmaxf(m_run, mx);
    const float p = (sc == -INFINITY) ? 0.f : expf(sc - m_new);
    const float alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
    float psum = p;
#pragma unroll
    for (int m = G; m < 64; m <<= 1) psum += __shfl_xor(psum, m);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    s_p[wave][lane] = p;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float al = __shfl(alpha, h);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= al;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = i * TPI + lane / LPT;
      float vf[8];
      unpack8(vr[i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pv = s_p[wave][t * G + h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv, vf[e], acc[h][e]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // --- combine the 4 waves (and the TPI token groups inside each wave)
  if (lane < G) { s_m[wave][lane] = m_run; s_l[wave][lane] = l_run; }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) s_acc[wave][h * 8 + e][lane] = acc[h][e];
  __syncthreads();

  const size_t qh0 = (size_t)b * Hq + (size_t)g * G;  // first query head row of this group
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx % D;
    const int dc = d / 8, e = d % 8;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_m[w][h];
      const float sc = (mw == -INFINITY) ? 0.f : expf(mw - M);
      L += s_l[w][h] * sc;
      float ow = 0.f;
#pragma unroll
      for (int grp = 0; grp < TPI; ++grp) ow += s_acc[w][h * 8 + e][grp * LPT + dc];
      o += ow * sc;
    }
    if (nsplit == 1) {
      a.out[(qh0 + h) * D + d] = o / L;
    } else {
      st_agent(a.o_part + ((qh0 + h) * S_max + s) * D + d, o);
      if (d == 0) {
        st_agent(a.ml_part + ((qh0 + h) * S_max + s) * 2 + 0, M);
        st_agent(a.ml_part + ((qh0 + h) * S_max + s) * 2 + 1, L);
      }
    }
  }
  if (nsplit == 1) return;

  unsigned* cnt = &a.counters[(size_t)b * Hkv + g];
  if (!arrive_last(cnt, (unsigned)nsplit, &s_flag)) return;
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx % D;
    const float* ml = a.ml_part + (qh0 + h) * S_max * 2;
    const float* op = a.o_part + (qh0 + h) * S_max * D + d;
    float M = -INFINITY;
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
      float mv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) mv[j] = ld_agent(ml + min(s0 + j, nsplit - 1) * 2);
#pragma unroll
      for (int j = 0; j < 8; ++j) M = fmaxf(M, mv[j]);
    }
    float L = 0.f, o = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
      float mv[8], lv[8], ov[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s2 = min(s0 + j, nsplit - 1);
        mv[j] = ld_agent(ml + s2 * 2);
        lv[j] = ld_agent(ml + s2 * 2 + 1);
        ov[j] = ld_agent(op + (size_t)s2 * D);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (s0 + j < nsplit) {
          const float sc = expf(mv[j] - M);
          L += lv[j] * sc;
          o += ov[j] * sc;
        }
      }
    }
    a.out[(qh0 + h) * D + d] = o / L;
  }
  if (tid == 0) reset_counter(cnt);
}

// ------------------------------------------------------------------ launchers

hipError_t launch_repack(const uint16_t* src, int rows, int K, uint16_t* dst, int tile_mul,
                         int tile_add, hipStream_t s) {
  const size_t n = (size_t)(rows / kTileRows) * (K / kTileCols) * 64;
  int grid = (int)((n + 255) / 256);
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(repack_kernel, dim3(grid), dim3(256), 0, s, src, rows, K, dst, tile_mul,
                     tile_add);
  return hipGetLastError();
}

hipError_t launch_bf16_to_f32(const uint16_t* src, float* dst, int n, hipStream_t s) {
  hipLaunchKernelGGL(bf16_to_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_embed(const EmbedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(const float* x, const float* ssq, const float* gain, int H,
                               int B, int Bmax, float eps, float* out, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(B), dim3(256), 0, s, x, ssq, gain, H, Bmax, eps,
                     out);
  return hipGetLastError();
}

static int gemv_nb(int B) {
  if (B <= 1) return 1;
  if (B <= 2) return 2;
  if (B <= 4) return 4;
  if (B <= 16) return 16;
  if (B <= 32) return 32;
  return 64;
}

size_t gemv_lds_bytes(int B, int kps) {
  const int nb = gemv_nb(B);
  const size_t ks = (size_t)kps * kTileCols;
  return nb >= 16 ? (size_t)nb * (ks + 8) * 2 * 2 : (size_t)nb * ks * 4;
}

template <int NB, int MODE>
static hipError_t launch_gemv_t(const GemvArgs& a, hipStream_t s) {
  static bool attr_set = false;
  const size_t lds = gemv_lds_bytes(a.B, a.kps);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<NB, MODE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = (a.N / kRowsPerGroup) * a.S;
  hipLaunchKernelGGL((gemv_kernel<NB, MODE>), dim3(grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_gemv_m(const GemvArgs& a, hipStream_t s) {
  switch (gemv_nb(a.B)) {
    case 1: return launch_gemv_t<1, MODE>(a, s);
    case 2: return launch_gemv_t<2, MODE>(a, s);
    case 4: return launch_gemv_t<4, MODE>(a, s);
    case 16: return launch_gemv_t<16, MODE>(a, s);
    case 32: return launch_gemv_t<32, MODE>(a, s);
    default: return launch_gemv_t<64, MODE>(a, s);
  }
}

hipError_t launch_gemv(const GemvArgs& a, int mode, hipStream_t s) {
  switch (mode) {
    case kStore: return launch_gemv_m<kStore>(a, s);
    case kResid: return launch_gemv_m<kResid>(a, s);
    case kSwiGLU: return launch_gemv_m<kSwiGLU>(a, s);
    default: return launch_gemv_m<kArgmax>(a, s);
  }
}

template <int D, int G>
static hipError_t launch_attention_t(const AttnArgs& a, hipStream_t s) {
  const int grid = a.B * a.Hkv * a.S_max;
  hipLaunchKernelGGL((attention_kernel<D, G>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int head_dim, int group, hipStream_t s) {
  if (head_dim == 128) {
    if (group == 4) return launch_attention_t<128, 4>(a, s);
    if (group == 2) return launch_attention_t<128, 2>(a, s);
    if (group == 1) return launch_attention_t<128, 1>(a, s);
  } else if (head_dim == 64) {
    if (group == 4) return launch_attention_t<64, 4>(a, s);
    if (group == 2) return launch_attention_t<64, 2>(a, s);
    if (group == 1) return launch_attention_t<64, 1>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qd
