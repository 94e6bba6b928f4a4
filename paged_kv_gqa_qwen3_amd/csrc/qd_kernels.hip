// HIP kernels of the decode step, written for CDNA4 (gfx950, wave64).
//
// Decode is memory bound: a step streams every weight once (the pages find
// bf16 GEMV to be the dominant cost of decode, "GPU 算子与执行优化", Part 2
// kernel table), so the kernels are organised around one rule: keep enough
// 16-byte loads in flight to saturate HBM, and do everything else (norms,
// RoPE, KV append, residual adds, SwiGLU, argmax) in the prologue or epilogue
// of the work item that already has the data on chip.
//
// Every piece of work is an "item" function (one GEMV row group x K split,
// one (sequence, KV head, split) of attention, one embedding row).  The same
// items run as one kernel per step stage here (captured in a hipGraph per
// batch size); the attention and embedding items also run inside the batch-1
// streaming kernel (qd_stream.h), which walks the whole step in one
// cooperative launch and resolves the dependencies between stages with
// counters.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "qd_device.h"

namespace qd {

// ------------------------------------------------------------------ repack

// Row-major [rows][K] bf16 -> tile-major (see qd_internal.h).  Source row r
// lands in packed row (r / blk) * stride + off + r % blk: blk = 16 with
// stride 16 stacks q|k|v at a row offset, blk = 8 with stride 16 puts gate
// rows in the first half of each packed row tile (off 0) and up rows in the
// second (off 8).  One thread moves one 16-byte run of 8 columns.
__global__ void repack_kernel(const uint16_t* __restrict__ src, int rows, int K,
                              uint16_t* __restrict__ dst, int blk, int stride, int off) {
  const int KT = K / kTileCols, K8 = K / 8;
  const size_t n = (size_t)rows * K8;
  for (size_t c = blockIdx.x * (size_t)blockDim.x + threadIdx.x; c < n;
       c += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(c / K8), k = (int)(c % K8) * 8;
    const int R = (r / blk) * stride + off + r % blk;
    const int lane = R % kTileRows + kTileRows * ((k % kTileCols) / 8);
    uint16_t* d = dst + ((size_t)(R / kTileRows) * KT + k / kTileCols) * kTileElems + lane * 8;
    *reinterpret_cast<u32x4*>(d) = *reinterpret_cast<const u32x4*>(src + (size_t)r * K + k);
  }
}

__global__ void bf16_to_f32_kernel(const uint16_t* __restrict__ src, float* __restrict__ dst,
                                   int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = __uint_as_float((unsigned)src[i] << 16);
}

__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) { embed_item(a, no_done(), blockIdx.x); }

// out[b][k] = x[b][k] * rsqrt(sum(ssq partials)/H + eps) * gain[k]
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const float* x, const float* ssq,
                                                           const float* gain, int H, int Bmax,
                                                           float eps, float* out) {
  const int b = blockIdx.x;
  __shared__ float s_inv;
  if (threadIdx.x == 0) {
    float ss = 0.f;
    for (int g = 0; g < H / kSsqRows; ++g) ss += ssq[(size_t)g * Bmax + b];
    s_inv = rsqrtf(ss / (float)H + eps);
  }
  __syncthreads();
  for (int k = threadIdx.x; k < H; k += blockDim.x)
    out[(size_t)b * H + k] = x[(size_t)b * H + k] * s_inv * gain[k];
}


// ------------------------------------------------------------------ L2 prefetch

__device__ unsigned g_prefetch_sink;

// Prefetching workgroup j (of p.n_wg, the first at workgroup index first_wg
// of this launch, so on XCD (first_wg + j) % 8): with the other prefetchers
// of its XCD it reads the weight tiles of the next launch's items that will
// run on that XCD (items x, x + 8, ...), with cached loads, so that they sit
// in that XCD's L2 when the next launch reads them.  The loads are folded
// into one word, stored only on a match no weights here produce.
__device__ inline void l2_prefetch(const L2Prefetch& p, int first_wg, int j) {
  constexpr int kInFlight = 8;
  const int x = (first_wg + j) % 8, per = p.n_wg / 8, jj = j / 8;
  const u32x4* const w = reinterpret_cast<const u32x4*>(p.w);
  const int nt = blockDim.x;
  unsigned acc = 0;
  for (int m = jj; x + 8 * m < p.items; m += per) {
    const int i = x + 8 * m;
    const int rg = i / p.S, s = i - rg * p.S;
    const int kt0 = s * p.kps, nk = min(p.KT, kt0 + p.kps) - kt0;
    if (nk <= 0) continue;
    const int n = nk * 64, total = p.rt * n;  // 16-byte pieces: per row tile, in the item
    for (int q0 = threadIdx.x; q0 < total; q0 += nt * kInFlight) {
      u32x4 v[kInFlight];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) {
        const int q = min(q0 + u * nt, total - 1), t = q / n;
        v[u] = w[((size_t)(rg * p.rt + t) * p.KT + kt0) * 64 + (q - t * n)];
      }
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (acc == 0x9e3779b9u) g_prefetch_sink = acc;
}

// Occupancy floor per batch width: four workgroups per CU for the fp32
// (batch 1) items, three for the MFMA items up to 32 columns (the LDS cap
// of their input slices allows three), two above.
// RPW 2: items of 128 rows, two row tiles per wave (rt = 8).
// Workgroups past the items prefetch the next launch's weights (a.pf).
template <int NB, int MODE, int RPW = 1>
__global__ __launch_bounds__(256, NB == 1 ? 4 : NB <= 32 ? 3 : 2) void gemv_kernel(GemvArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int items = a.N / (kTileRows * a.rt) * a.S;
  if ((int)blockIdx.x >= items) {
    l2_prefetch(a.pf, items, (int)blockIdx.x - items);
    return;
  }
  gemv_item<NB, MODE, kMaxTilesInFlight, NoWait, RPW>(a, a.w, a.gain, no_done(), blockIdx.x, smem,
                                                      NoWait{});
}


// 32 and 64 batch columns: items of 64 * RW rows that stream their input
// slice through LDS in chunks (gemv_wide_item).
template <int NB, int MODE, int RW>
__global__ __launch_bounds__(256, 2) void gemv_wide_kernel(GemvArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int items = a.N / (kTileRows * a.rt) * a.S;
  if ((int)blockIdx.x >= items) {  // prefetching workgroups (a.pf)
    l2_prefetch(a.pf, items, (int)blockIdx.x - items);
    return;
  }
  gemv_wide_item<NB, MODE, RW>(a, no_done(), blockIdx.x, smem);
}

// The workgroups take the step's attention items round robin; workgroups
// past a.grid prefetch the next launch's weights (a.pf).
template <int D, int G, int NW, int PW, class KV>
__global__ __launch_bounds__(NW * 64) void attention_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  if ((int)blockIdx.x >= a.grid) {
    l2_prefetch(a.pf, a.grid, (int)blockIdx.x - a.grid);
    return;
  }
  const AttnList list = attn_list<NW * PW>(a);
  const int items = attn_items(list, a.B);
#ifdef QD_STEP_TRACE
  AttnArgs at = a;  // (trace builds) 8 event slots per workgroup
  if (a.trace != nullptr) at.trace = a.trace + (size_t)blockIdx.x * 8;
#else
  const AttnArgs& at = a;
#endif
  for (int t = blockIdx.x; t < items; t += a.grid)
    attention_item<D, G, NW, PW, NoWait, KV>(
        at, list, a.q_gain, a.k_gain, reinterpret_cast<typename KV::Elem*>(a.pool_layer),
        no_done(), t, smem, NoWait{});
}


// ------------------------------------------------------------------ fused layer launches

// Occupancy floor of the fused MLP launch: the GEMV items' (three
// workgroups per CU up to 32 batch columns).
constexpr int fused_min_blocks(int NB) { return NB == 1 ? 4 : 3; }

// The MLP half of one layer (see FusedMlpArgs): [gate/up items | down
// items] by workgroup index.  Gate/up items sit at lower indices, which are
// dispatched first, so a waiting down item only waits for running or
// finished workgroups; each wait is bounded besides.  (A grid of resident
// workgroups that each run their gate/up items and then their down items
// was measured slower: batch 8, 3.56 against 2.97 ms per step; down's early
// weight loads slowed gate/up's without shortening the block.)
template <int NB, int RG = 1, int RD = 1>  // row tiles per wave of gate/up and of down items
__global__ __launch_bounds__(256, fused_min_blocks(NB)) void fused_mlp_kernel(FusedMlpArgs f) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int wg = blockIdx.x;
  if (wg >= f.ng + f.nd) {
    l2_prefetch(f.pf, f.ng + f.nd, wg - f.ng - f.nd);
    return;
  }
  if (wg == 0)  // the next launch's counters
    for (int i = threadIdx.x; i < f.n_other; i += blockDim.x)
      st_agent(f.cnt_other + (size_t)i * kCntStride, 0u);
  const int rows_gu = kTileRows * f.gu.rt;
  if (wg < f.ng) {
    // a gate/up row group yields rows/2 SwiGLU channels: down k-tile
    // rg * rows/2 / 32, in down's K slice (that) / kps
    const int rg = wg / f.gu.S;
    const int sd = (rg * (rows_gu / 2) / kTileCols) / f.d.kps;
    gemv_item<NB, kSwiGLU, kMaxTilesInFlight, NoWait, RG>(
        f.gu, f.gu.w, f.gu.gain, Done{f.cnt_g + (size_t)sd * kCntStride, 0u, 0u, nullptr, 0}, wg,
        smem, NoWait{});
    return;
  }
  // down item: waits for the gate/up row groups that feed its K slice
  const int item = wg - f.ng;
  const int s = item % f.d.S;
  const int KT = f.d.K / kTileCols;
  const int nk = min(KT, (s + 1) * f.d.kps) - s * f.d.kps;
  const unsigned target = (unsigned)(nk * kTileCols / (rows_gu / 2));
  gemv_item<NB, kResid, kMaxTilesInFlight, CounterWait, RD>(
      f.d, f.d.w, nullptr, no_done(), item, smem,
      CounterWait{f.cnt_g + (size_t)s * kCntStride, 1, target, f.dev_flags, f.spin_limit});
}

// ------------------------------------------------------------------ read ceiling

// A plain streaming read, the measured ceiling of the weight-streaming
// pattern: every wave reads its contiguous share of the buffer in 1 KB
// pieces (one 16-byte nontemporal load per lane), kMaxTilesInFlight pieces
// in flight, refilling each register set as soon as it has been folded into
// one word (the loads stay live; the word is stored only on a match no
// buffer here produces).
__device__ unsigned g_read_sink;

__global__ __launch_bounds__(256) void read_ceiling_kernel(const u32x4* __restrict__ src,
                                                           size_t pieces) {
  constexpr int CH = kMaxTilesInFlight;
  const int lane = threadIdx.x & 63;
  const size_t nw = (size_t)gridDim.x * 4;
  const size_t w = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t per = (pieces + nw - 1) / nw;
  const size_t p0 = w * per, p1 = p0 + per < pieces ? p0 + per : pieces;
  if (p0 >= p1) return;
  const size_t n = p1 - p0, last = n - 1;
  const u32x4* q = src + p0 * 64 + lane;
  unsigned acc = 0;
  u32x4 buf[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) buf[i] = __builtin_nontemporal_load(q + min((size_t)i, last) * 64);
  size_t c0 = 0;
  for (; c0 + CH < n; c0 += CH) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      acc ^= buf[i].x ^ buf[i].y ^ buf[i].z ^ buf[i].w;
      buf[i] = __builtin_nontemporal_load(q + min(c0 + CH + i, last) * 64);
    }
  }
#pragma unroll
  for (int i = 0; i < CH; ++i)
    if (c0 + i < n) acc ^= buf[i].x ^ buf[i].y ^ buf[i].z ^ buf[i].w;
  if (acc == 0x9e3779b9u) g_read_sink = acc;
}

// ------------------------------------------------------------------ launchers

bool fused_supported(int B) {
  const int nb = gemv_nb(B);
  return nb == 8 || nb == 16;
}

template <int NB, int RG, int RD>
static hipError_t launch_fused_mlp_t(const FusedMlpArgs& a, size_t lds, hipStream_t s) {
  static bool attr_set = false;
  const void* fn = reinterpret_cast<const void*>(&fused_mlp_kernel<NB, RG, RD>);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int pf = a.pf.w != nullptr ? a.pf.n_wg : 0;
  hipLaunchKernelGGL((fused_mlp_kernel<NB, RG, RD>), dim3(a.ng + a.nd + pf), dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_fused_mlp(const FusedMlpArgs& a, size_t lds, hipStream_t s) {
  switch (gemv_nb(a.gu.B)) {
    case 8: return launch_fused_mlp_t<8, 1, 1>(a, lds, s);
    case 16:
      if (a.gu.rt == 8)
        return a.d.rt == 8 ? launch_fused_mlp_t<16, 2, 2>(a, lds, s) : launch_fused_mlp_t<16, 2, 1>(a, lds, s);
      return a.d.rt == 8 ? launch_fused_mlp_t<16, 1, 2>(a, lds, s) : launch_fused_mlp_t<16, 1, 1>(a, lds, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_read_ceiling(const void* src, size_t bytes, int grid, hipStream_t s) {
  hipLaunchKernelGGL(read_ceiling_kernel, dim3(grid), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), bytes / 1024);
  return hipGetLastError();
}

hipError_t launch_repack(const uint16_t* src, int rows, int K, uint16_t* dst, int blk,
                         int stride, int off, hipStream_t s) {
  const size_t n = (size_t)rows * (K / 8);
  int grid = (int)((n + 255) / 256);
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(repack_kernel, dim3(grid), dim3(256), 0, s, src, rows, K, dst, blk, stride,
                     off);
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

template <int NB, int MODE, int RPW = 1>
static hipError_t launch_gemv_t(const GemvArgs& a, hipStream_t s) {
  static bool attr_set = false;
  const size_t lds = gemv_lds_bytes(a.B, a.kps, a.rt);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_kernel<NB, MODE, RPW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = (a.N / (kTileRows * a.rt)) * a.S + (a.pf.w != nullptr ? a.pf.n_wg : 0);
  hipLaunchKernelGGL((gemv_kernel<NB, MODE, RPW>), dim3(grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int NB, int MODE, int RW>
static hipError_t launch_wide_t(const GemvArgs& a, hipStream_t s) {
  static bool attr_set = false;
  const void* fn = reinterpret_cast<const void*>(&gemv_wide_kernel<NB, MODE, RW>);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = (a.N / (kTileRows * a.rt)) * a.S + (a.pf.w != nullptr ? a.pf.n_wg : 0);
  hipLaunchKernelGGL((gemv_wide_kernel<NB, MODE, RW>), dim3(grid), dim3(256),
                     gemv_wide_lds_bytes(NB, RW), s, a);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_gemv_m(const GemvArgs& a, hipStream_t s) {
  if (a.wide) {  // chunk-streamed items of 128 rows
    switch (gemv_nb(a.B)) {
      case 8:
      case 16: return launch_wide_t<16, MODE, 2>(a, s);
      case 32: return launch_wide_t<32, MODE, 2>(a, s);
      case 64: return launch_wide_t<64, MODE, 2>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (gemv_nb(a.B)) {
    case 1: return launch_gemv_t<1, MODE>(a, s);
    case 8: return launch_gemv_t<8, MODE>(a, s);
    case 16:
      if (a.rt == 8) return launch_gemv_t<16, MODE, 2>(a, s);
      return launch_gemv_t<16, MODE>(a, s);
    case 32: return launch_gemv_t<32, MODE>(a, s);
    default: return launch_gemv_t<64, MODE>(a, s);
  }
}

hipError_t launch_gemv(const GemvArgs& a, int mode, hipStream_t s) {
  switch (mode) {
    case kStore: return launch_gemv_m<kStore>(a, s);
    case kResid: return launch_gemv_m<kResid>(a, s);
    case kSwiGLU: return launch_gemv_m<kSwiGLU>(a, s);
    case kPartial: return launch_gemv_m<kPartial>(a, s);
    default: return launch_gemv_m<kArgmax>(a, s);
  }
}

template <int D, int G, int NW, int PW, class KV>
static hipError_t launch_attention_t(const AttnArgs& a, hipStream_t s) {
  const int pf = a.pf.w != nullptr ? a.pf.n_wg : 0;
  hipLaunchKernelGGL((attention_kernel<D, G, NW, PW, KV>), dim3(a.grid + pf), dim3(NW * 64),
                     sizeof(AttnSmem<D, G, NW, PW>), s, a);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_attention_dg(const AttnArgs& a, int pages, hipStream_t s) {
  if (!a.kv_fp8) {
    if (pages == 1) return launch_attention_t<D, G, kAttnWaves, 1, KvBf16>(a, s);
    if (pages == 2) return launch_attention_t<D, G, kAttnWaves, 2, KvBf16>(a, s);
    if (pages == 3) return launch_attention_t<D, G, kAttnWaves, 3, KvBf16>(a, s);
  } else {
    if (pages == 2) return launch_attention_t<D, G, kAttnWaves, 2, KvFp8>(a, s);
    if (pages == 5) return launch_attention_t<D, G, kAttnWaves, 5, KvFp8>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention(const AttnArgs& a, int head_dim, int group, int waves, int pages,
                            hipStream_t s) {
  if (waves != kAttnWaves) return hipErrorInvalidValue;  // (pages: launch_attention_dg)
  if (head_dim == 128) {
    if (group == 4) return launch_attention_dg<128, 4>(a, pages, s);
    if (group == 2) return launch_attention_dg<128, 2>(a, pages, s);
    if (group == 1) return launch_attention_dg<128, 1>(a, pages, s);
  } else if (head_dim == 64) {
    if (group == 4) return launch_attention_dg<64, 4>(a, pages, s);
    if (group == 2) return launch_attention_dg<64, 2>(a, pages, s);
    if (group == 1) return launch_attention_dg<64, 1>(a, pages, s);
  }
  return hipErrorInvalidValue;
}

size_t gemv_lds_bytes(int B, int kps, int rt) { return gemv_lds_bytes_impl(B, kps, rt); }

}  // namespace qd
