// The batch-1 decode step as one persistent cooperative kernel that streams
// weights continuously (included by qd_stream.hip).
//
// At batch 1 every projection is one of a chain of dependent stages, and each
// stage boundary costs a few microseconds of hand-off latency (stores
// performed, completion counted, waiting workgroups released).  If the
// weights of a stage only started to stream once its input was ready, HBM
// would idle for every one of those hand-offs.  Here every wave owns a fixed
// share of every projection's weight tiles (its workgroup's row tiles, every
// 4th k-tile of each) and streams them in step order into a private ring of
// kStreamRing 1 KB slots in LDS with direct global-to-LDS loads, as far ahead as the
// ring allows and independently of the stage it is computing: while a
// workgroup waits for a stage's input its rings hold the next tiles it will
// need.  The compute side consumes the ring in the same order.
//
// Each 1 KB weight tile is two 16x16x32 bf16 MFMAs against the input split
// into a bf16 pair (hi = bf16(x), lo = bf16(x - hi), about 16 significant
// bits), the input broadcast to all 16 columns: a wave runs alone on its
// SIMD, where every instruction costs an issue slot, and this takes 5
// instructions per tile (one ring read, two input reads, two MFMAs) where
// unpacking and FMAs in fp32 take over 20.  Attention is the item function
// of the per-stage kernels.
#pragma once

#include "qd_device.h"
#include "qd_stream_plan.h"

namespace qd {

// 4-float groups of a staged input per thread: inputs up to 16384 floats.
constexpr int kStageVec = kStreamStageVec;
// ... and of an RMSNorm gain (the hidden size: at most 8192 floats).
constexpr int kGainVec = 8;


// The wave's ring: its slots, the loader (position and counts) and the
// slot the consumer reads next.
struct StreamRing {
  unsigned char* slots;  // kStreamRing slots of 1 KB
  StreamLoader ld;
  int cs_slot;
  int W, wg;             // grid size and this workgroup
#ifdef QD_STEP_TRACE
  unsigned long long t_wait, t_dot;  // (trace builds) shader cycles waiting for tiles / in ring_mfma
  unsigned long long t_top, t_rel;   // ... refilling / waiting for a batch's LDS reads
#endif
};

// Top the ring up (stream_refill) with direct global-to-LDS loads: lane l's
// 16 bytes of a tile land at byte 16*l of its slot, i.e. in the order of
// the packed tile.
__device__ __forceinline__ void ring_top_up(const StreamArgs& a, StreamRing& rg, int wave,
                                            int lane, int u_limit) {
  unsigned char* const slots = rg.slots;
  stream_refill(rg.ld, u_limit, [&](const unsigned char* tile, int slot) {
                  __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4*>(tile) + lane,
                                                   slots + (size_t)slot * 1024, 16, 0,
                                                   kNonTemporal);
                });
}

// Wait until the next N (1..kBatch) tiles of the ring have landed.  A
// wave's vector-memory loads complete in issue order, so they are in LDS
// once at most (loads issued after them) operations are outstanding; any
// other memory operation issued since only makes the wait stricter.
template <int N>
__device__ __forceinline__ void ring_wait(const StreamRing& rg) {
  static_assert(N >= 1 && N <= kBatch, "batch size");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (rg.ld.issued - rg.ld.consumed == kStreamRing)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kStreamRing - N));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// This lane's 16 bytes of the i-th unconsumed tile.
__device__ __forceinline__ u32x4 ring_read(const StreamRing& rg, int i, int lane) {
  int slot = rg.cs_slot + i;
  if (slot >= kStreamRing) slot -= kStreamRing;
  return *reinterpret_cast<const u32x4*>(rg.slots + (size_t)slot * 1024 + lane * 16);
}

// The next n tiles have been read (their LDS reads completed): their slots
// may be refilled.
__device__ __forceinline__ void ring_release(StreamRing& rg, int n) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kLgkmZero);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  rg.ld.consumed += n;
  rg.cs_slot += n;
  if (rg.cs_slot >= kStreamRing) rg.cs_slot -= kStreamRing;
}

// Accumulators of a wave's 16-row tile sums.  The input's bf16 pair is
// spread over the MFMA's 16 columns: the lanes of columns 0..7 supply hi,
// those of columns 8..15 lo, so that one MFMA per tile yields both products
// (columns 0..7 hold W*hi, 8..15 W*lo); kBatch accumulators keep the MFMAs of
// a batch independent.  Lane l holds rows 4*(l/16) .. +3 of column l % 16.
struct Acc2 {
  f32x4 a[kBatch];
  __device__ __forceinline__ Acc2() {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) a[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // W*(hi + lo) of the lane's 4 rows, the same in all 16 lanes of a row
  // group (every lane takes part: a column's partner is lane ^ 8)
  __device__ __forceinline__ f32x4 total() const {
    f32x4 t = a[0];
#pragma unroll
    for (int i = 1; i < kBatch; ++i) t += a[i];
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = t[e] + __shfl_xor(t[e], 8);
    return r;
  }
};

// This lane's input column pointer: hi for columns 0..7, lo for 8..15 (the
// pair is hi [K] then lo [K]), at k-group lane / 16 of a tile.
__device__ __forceinline__ const unsigned short* stream_in_lane(const unsigned short* xsh, int K,
                                                               int lane) {
  return xsh + ((lane & 8) ? K : 0) + (lane >> 4) * 8;
}

__device__ __forceinline__ f32x4 tile_mfma(u32x4 w, u32x4 x, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w),
                                                 __builtin_bit_cast(bf16x8, x), acc, 0, 0, 0);
}

// acc += the next tile of the stream against the input at xk (this lane's
// 16 bytes of it); the freed slot is refilled before the arithmetic.
__device__ __forceinline__ void ring_mfma1(const StreamArgs& a, StreamRing& rg, int wave, int lane,
                                           int u_limit, const unsigned short* xk, Acc2& acc) {
#ifdef QD_STEP_TRACE
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
#endif
  ring_top_up(a, rg, wave, lane, u_limit);
#ifdef QD_STEP_TRACE
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
#endif
  ring_wait<1>(rg);
#ifdef QD_STEP_TRACE
  rg.t_wait += __builtin_amdgcn_s_memtime() - t1;
#endif
  const u32x4 w = ring_read(rg, 0, lane);
  const u32x4 x = *reinterpret_cast<const u32x4*>(xk);
  ring_release(rg, 1);
  ring_top_up(a, rg, wave, lane, u_limit);
  acc.a[0] = tile_mfma(w, x, acc.a[0]);
#ifdef QD_STEP_TRACE
  rg.t_dot += __builtin_amdgcn_s_memtime() - t0;
#endif
}

// One batch of kBatch tiles as read from LDS: this lane's 16 bytes of each
// weight tile and of its input columns.
struct StreamBatch {
  u32x4 w[kBatch], x[kBatch];
};

// Issue the LDS reads of the batch at the consumer's next kBatch slots, the
// tiles' inputs at xk + i * KSTEP k-tiles.  Slots that do not wrap around the
// ring are addressed from one base with immediate offsets.
template <int KSTEP>
__device__ __forceinline__ void batch_read(const StreamRing& rg, int lane,
                                           const unsigned short* xk, StreamBatch& bt) {
  if (rg.cs_slot <= kStreamRing - kBatch) {
    const unsigned char* base = rg.slots + (size_t)rg.cs_slot * 1024 + lane * 16;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) bt.w[i] = *reinterpret_cast<const u32x4*>(base + i * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) bt.w[i] = ring_read(rg, i, lane);
  }
#pragma unroll
  for (int i = 0; i < kBatch; ++i)
    bt.x[i] = *reinterpret_cast<const u32x4*>(xk + i * KSTEP * kTileCols);
}

__device__ __forceinline__ void batch_mfma(const StreamBatch& bt, Acc2& acc) {
#pragma unroll
  for (int i = 0; i < kBatch; ++i) acc.a[i] = tile_mfma(bt.w[i], bt.x[i], acc.a[i]);
}

// acc += tiles j = 0 .. n-1 of the stream, tile j against the input at
// xk + j * KSTEP k-tiles.  Full batches are software-pipelined over two
// register sets: the next batch's wait and LDS reads are issued before the
// current batch's MFMAs, so that the LDS round trip overlaps them and the
// refill; the tail goes one tile at a time.
template <int KSTEP>
__device__ __forceinline__ void ring_mfma_run(const StreamArgs& a, StreamRing& rg, int wave,
                                              int lane, int u_limit, int n,
                                              const unsigned short* xk, Acc2& acc) {
  constexpr int kStep = kBatch * KSTEP * kTileCols;  // input elements between batches
  const int nfull = n / kBatch;
  if (nfull > 0) {
#ifdef QD_STEP_TRACE
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
#endif
    StreamBatch A, B;
    ring_top_up(a, rg, wave, lane, u_limit);
    ring_wait<kBatch>(rg);
    batch_read<KSTEP>(rg, lane, xk, A);
    // batches 2p (in A) and 2p + 1 (in B)
#ifdef QD_STEP_TRACE
    // (trace builds) shader cycles spent waiting for tiles, releasing, refilling
    auto timed_wait = [&]() {
      const unsigned long long tw = __builtin_amdgcn_s_memtime();
      ring_wait<kBatch>(rg);
      rg.t_wait += __builtin_amdgcn_s_memtime() - tw;
    };
    auto rel_top = [&]() {
      const unsigned long long t0 = __builtin_amdgcn_s_memtime();
      ring_release(rg, kBatch);
      const unsigned long long t1 = __builtin_amdgcn_s_memtime();
      ring_top_up(a, rg, wave, lane, u_limit);
      const unsigned long long t2 = __builtin_amdgcn_s_memtime();
      rg.t_rel += t1 - t0;
      rg.t_top += t2 - t1;
    };
#else
    auto timed_wait = [&]() { ring_wait<kBatch>(rg); };
    auto rel_top = [&]() {
      ring_release(rg, kBatch);
      ring_top_up(a, rg, wave, lane, u_limit);
    };
#endif
    for (int p = 0; p < nfull / 2; ++p) {
      rel_top();  // (the release waits for batch 2p's reads)
      timed_wait();
      batch_read<KSTEP>(rg, lane, xk + (2 * p + 1) * kStep, B);
      batch_mfma(A, acc);
      rel_top();  // (waits for batch 2p + 1's reads)
      if (2 * p + 2 < nfull) {
        timed_wait();
        batch_read<KSTEP>(rg, lane, xk + (2 * p + 2) * kStep, A);
      }
      batch_mfma(B, acc);
    }
    if (nfull & 1) {  // the last batch, in A
      ring_release(rg, kBatch);
      ring_top_up(a, rg, wave, lane, u_limit);
      batch_mfma(A, acc);
    }
#ifdef QD_STEP_TRACE
    rg.t_dot += __builtin_amdgcn_s_memtime() - t0;
#endif
  }
  for (int j = nfull * kBatch; j < n; ++j)
    ring_mfma1(a, rg, wave, lane, u_limit, xk + j * KSTEP * kTileCols, acc);
}

// Wait until the step reached `phase` (every wave polls its workgroup's
// flag, topping up its ring meanwhile).  Bounded like Waiter: after
// spin_limit polls it records QD_DEV_TIMEOUT and sets the abort flag, after
// which every later wait falls through.
__device__ __forceinline__ void stream_wait(const StreamArgs& a, StreamRing& rg, int wave, int lane,
                                   unsigned phase, int u_limit) {
  const unsigned* flag = a.flags + (size_t)blockIdx.x * kFlagStride;
  ring_top_up(a, rg, wave, lane, u_limit);
  // the flag values are read into scalar registers, so that the loop (and
  // the ring state it updates) stays uniform across the wave
  for (unsigned n = 0;; ++n) {
    if (__builtin_amdgcn_readfirstlane(ld_agent(flag)) >= phase) break;
    ring_top_up(a, rg, wave, lane, u_limit);
    if ((n & 63) == 0 && __builtin_amdgcn_readfirstlane(ld_agent(a.abort_flag)) != 0u) break;
    if (n >= a.spin_limit) {
      if (lane == 0) set_flag(a.dev_flags, QD_DEV_TIMEOUT);
      st_agent(a.abort_flag, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Completion of this workgroup's share of a stage.  Only wave 0 stores
// results, so only it waits for its stores to be performed (its ring holds
// no load beyond the stage it just finished, see stream_step_kernel); then
// the counter and, from the last workgroup to arrive, every flag.
__device__ __forceinline__ void stream_signal(const Done& d, unsigned* s_last) {
  if ((threadIdx.x >> 6) == 0) stores_done();
  lds_barrier();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(d.counter, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    *s_last = prev + 1 == d.target ? 1u : 0u;
  }
  lds_barrier();
  if (*s_last != 0u)
    for (int i = threadIdx.x; i < d.nflags; i += blockDim.x)
      __hip_atomic_fetch_max(d.flags + (size_t)i * kFlagStride, d.phase, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// LDS after the rings: the stage input (first in fp32 as loaded, then as
// its bf16 pair: hi [K] and lo [K]) and the old residual of the
// workgroup's rows at float offset res_off (or an attention item's LDS,
// never live at the same time), then the waves' row sums (rt_max row tiles
// x 4 waves x 16 rows) and a few scalars.
struct StreamMisc {
  float s_ssq[4];
  unsigned s_last;
  float amax_v[4];
  int amax_i[4];
  float tmp[8];
};

template <int D, int G>
constexpr size_t stream_in_bytes_t(int in_floats) {
  const size_t x = (size_t)in_floats * 4;
  const size_t att = sizeof(AttnSmem<D, G, kAttnWavesPersistent, attn_pages_per_wave(1, true)>);
  return ((x > att ? x : att) + 15) / 16 * 16;
}

template <int D, int G>
constexpr size_t stream_lds_bytes_t(int in_floats, int rt_max) {
  return (size_t)4 * kStreamRing * 1024 + stream_in_bytes_t<D, G>(in_floats) +
         (size_t)rt_max * 4 * kTileRows * 4 + sizeof(StreamMisc);
}

template <int D, int G>
__global__ __launch_bounds__(256) void stream_step_kernel(const StreamArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = gridDim.x, wg = blockIdx.x;
  const int u_end = a.L * kUnitsPerLayer + 1;
  unsigned char* in_lds = smem + (size_t)4 * kStreamRing * 1024;
  float* xs = reinterpret_cast<float*>(in_lds);
  float* red = reinterpret_cast<float*>(in_lds + stream_in_bytes_t<D, G>(a.in_floats));
  StreamMisc& sm = *reinterpret_cast<StreamMisc*>(red + (size_t)a.rt_max * 4 * kTileRows);

  // Wave 0 stores every stage's results and must then wait for its stores,
  // which also waits for every load it issued before them: its ring never
  // runs ahead of the unit it computes or waits for (u_lim), so that wait
  // costs no more than the stores.  The other waves stream ahead freely.
  StreamRing rg;
  rg.slots = smem + (size_t)wave * kStreamRing * 1024;
  rg.cs_slot = 0;
  rg.W = W;
  rg.wg = wg;
#ifdef QD_STEP_TRACE
  rg.t_wait = rg.t_dot = rg.t_top = rg.t_rel = 0;
#endif
  stream_start(rg.ld, a.runs + __builtin_amdgcn_readfirstlane(a.run_off[wg * 4 + wave]));
  auto u_lim = [&](int u) { return wave == 0 ? u : u_end; };
  ring_top_up(a, rg, wave, lane, u_lim(0));

  auto done = [&](int i, unsigned target) {
    return Done{a.cnt + i, target, (unsigned)i + 1u, a.flags, W};
  };
#ifdef QD_STEP_TRACE
  // (trace builds) event e of this workgroup: 100 MHz clock, from thread 0
  auto mark = [&](int e) {
    if (tid == 0) a.trace[(size_t)wg * 1024 + e] = __builtin_amdgcn_s_memrealtime();
    // ... and wave 1's time and weight tiles issued so far, in two more blocks
    if (tid == 64) {
      a.trace[(size_t)gridDim.x * 1024 + (size_t)wg * 1024 + e] = __builtin_amdgcn_s_memrealtime();
      a.trace[(size_t)gridDim.x * 2048 + (size_t)wg * 1024 + e] = (unsigned long long)rg.ld.issued;
    }
  };
#else
  auto mark = [](int) {};
#endif
  mark(1023);
  auto phase = [](int i) { return (unsigned)i + 1u; };

  // embedding (workgroup 0)
  if (wg == 0) embed_item(a.embed, done(kCntEmbed, 1u), 0);

  // The input of a projection in LDS as the bf16 pair of x (times the
  // RMSNorm gain), 1/rms of it from the producer's partial sums of squares
  // (s_inv, the same in every thread) and, for a residual epilogue, the old
  // residual of the workgroup's row tiles [r0, r1) at xres.  Every thread
  // loads its own 4-float groups with device-scope 16-byte loads (the data
  // was written in this launch; past the end they return zeros).
  float* const xres = xs + a.res_off;
  unsigned short* const xsh = reinterpret_cast<unsigned short*>(xs);
  float s_inv = 1.f;
  auto stage_input = [&](const float* in, int K, const float* gain, int r0, int r1) {
    const bool norm = gain != nullptr;
    const int nj = (K + 1023) / 1024;
    const __amdgpu_buffer_rsrc_t rin =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(in), 0, K * 4, kBufferWord3);
    f32x4 xv[kStageVec], gv[kGainVec];
#pragma unroll
    for (int j = 0; j < kStageVec; ++j) {
      if (j < nj) {
        xv[j] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rin, 16 * (tid + 256 * j), 0, kDeviceScope));
        if (norm && j < kGainVec)  // (under a norm K is the hidden size: j < kGainVec)
          gv[j] = *reinterpret_cast<const f32x4*>(gain + min(4 * (tid + 256 * j), K - 4));
      }
    }
    for (int i = tid; i < (r1 - r0) * kTileRows; i += 256)
      xres[i] = ld_agent(a.x + r0 * kTileRows + i);
    if (norm) {
      const int ng = K / kSsqRows;
      float ss = 0.f;
      for (int g = tid; g < ng; g += 256) ss += ld_agent(a.ssq + (size_t)g * a.Bmax);
      ss = wave_sum(ss);
      if (lane == 0) sm.s_ssq[wave] = ss;
    }
#pragma unroll
    for (int j = 0; j < kStageVec; ++j) {
      const int i = 4 * (tid + 256 * j);
      if (j < nj && i < K) {
        f32x4 v = xv[j];
        if (norm && j < kGainVec) v *= gv[j];
        unsigned short h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[e] = f2bf(v[e]);
          l[e] = f2bf(v[e] - __uint_as_float((unsigned)h[e] << 16));
        }
        *reinterpret_cast<uint2*>(xsh + i) =
            make_uint2(h[0] | ((unsigned)h[1] << 16), h[2] | ((unsigned)h[3] << 16));
        *reinterpret_cast<uint2*>(xsh + K + i) =
            make_uint2(l[0] | ((unsigned)l[1] << 16), l[2] | ((unsigned)l[3] << 16));
      }
    }
    lds_barrier();
    if (norm)
      s_inv = rsqrtf((sm.s_ssq[0] + sm.s_ssq[1] + sm.s_ssq[2] + sm.s_ssq[3]) / (float)K + a.eps);
  };

  // The workgroup's pieces of unit u: every wave adds its k-tiles of each
  // piece (k-tiles kb + wave, kb + wave + 4, ...) and leaves the 16 row sums
  // in red[piece][wave]; then wave 0 adds the waves in K order, scales by
  // 1/rms under RMSNorm and runs epi(piece in the workgroup, piece, y) with
  // 16 lanes per piece (lane: row lane % 16).  Without a K split a piece is
  // a row tile.
  auto project = [&](int u, int u_limit, bool norm, auto&& epi) {
    const StreamShare s = stream_share(a, u, wave, W, wg);
    const unsigned short* const xin = stream_in_lane(xsh, s.KT * kTileCols, lane);
    for (int r = s.r0; r < s.r1; ++r) {
      int kb, ke;
      stream_piece(s, r, kb, ke);
      Acc2 acc;
      ring_mfma_run<kStreamKStep>(a, rg, wave, lane, u_limit, stream_piece_tiles(s, r),
                                  xin + (kb + s.kstart) * kTileCols, acc);
      const f32x4 t = acc.total();
      if ((lane & 15) == 0)
        *reinterpret_cast<f32x4*>(red + ((r - s.r0) * 4 + wave) * kTileRows + (lane >> 4) * 4) = t;
    }
    lds_barrier();
    if (wave == 0) {
      for (int rr = lane >> 4; rr < s.r1 - s.r0; rr += 4) {
        const float* rp = red + (size_t)rr * 4 * kTileRows + (lane & 15);
        float y = rp[0];
        for (int w2 = 1; w2 < 4; ++w2) y += rp[w2 * kTileRows];
        if (norm) y *= s_inv;
        epi(rr, s.r0 + rr, y);
      }
    }
  };

  // residual epilogue: x += y, and the sum of squares of each 16 new rows
  auto resid = [&](int rr, int rt, float y) {
    const int n = rt * kTileRows + (lane & 15);
    const float xv = xres[rr * kTileRows + (lane & 15)] + y;
    st_agent(a.x + n, xv);
    const float ss = group_sum(xv * xv, kSsqRows);
    if ((lane & 15) == 0) st_agent(a.ssq + (size_t)(n / kSsqRows) * a.Bmax, ss);
  };

  // Stage taps (checking only): workgroup 0 copies a stage's result out
  // once every workgroup has finished that stage (it is read here before
  // workgroup 0 itself finishes the next stage, so nothing overwrites it).
  auto tap_copy = [&](float* dst, const float* src, int n) {
    if (dst != nullptr && wg == 0)
      for (int i = tid; i < n; i += 256) dst[i] = ld_agent(src + i);
  };

  const unsigned n_heads = (unsigned)a.attn.Hkv;
  const AttnList alist = attn_list<attn_pages_per_split(1, true)>(a.attn);
  const int attn_n = __builtin_amdgcn_readfirstlane(attn_items(alist, 1));
  // Attention items go to workgroups that own no row of the O projection
  // (so no O tiles wait for them meanwhile), when there are enough of those
  // (4B shape: 96 of 256; batch 1, context 512: 2.374 -> 2.358 ms per step
  // against items on workgroups 0..71).  Ownership is decided on the
  // XCD-major place (stream_place), which spreads the idle workgroups, like
  // every unit's pieces, evenly over the XCDs (2.354 -> 2.343 ms per step
  // against the plain order, where O owners sat on 5 of the 8 XCDs).
  const unsigned R_o = (unsigned)(a.H / kTileRows);
  const int n_idle = (unsigned)W > R_o ? W - (int)R_o : 0;
  const int wq = stream_place(wg, W);
  const int o_before = (int)((unsigned)wq * R_o / (unsigned)W);
  const bool o_idle = (int)((unsigned)(wq + 1) * R_o / (unsigned)W) == o_before;
  const int a_first = n_idle >= attn_n ? (o_idle ? wq - o_before : attn_n) : wg;
  const bool attn_wg = a_first < attn_n;  // this workgroup runs attention items

  for (int l = 0; l < a.L; ++l) {
    const LayerDev ly = a.layers[l];
    const int c = cnt_index(l, 0);
    const int u = l * kUnitsPerLayer;
    const unsigned x_ready = l == 0 ? phase(kCntEmbed) : phase(cnt_index(l - 1, 4));

    // QKV, as qkv_S split partials per row that attention sums.  A
    // workgroup that runs attention items loads no tile past the
    // QKV unit meanwhile: its K/V page loads, issued when its item starts,
    // would otherwise complete only after those tiles (loads complete in
    // order); it fetches its next tiles while it waits for the other items.
    const int lim_qkv = attn_wg ? u + kPrQkv : u_lim(u + kPrQkv);
    stream_wait(a, rg, wave, lane, x_ready, lim_qkv);
    mark(l * 20 + 0);
    if (l == a.tap_layer) tap_copy(a.tap_x_in, a.x, a.H);
    if (l - 1 == a.tap_layer) tap_copy(a.tap_x_out, a.x, a.H);
    stage_input(a.x, a.H, ly.in_norm, 0, 0);
    mark(l * 20 + 1);
    project(u + kPrQkv, lim_qkv, true, [&](int, int piece, float y) {
      st_agent(a.qkv_part + piece * kTileRows + (lane & 15), y);  // = [rt][split][row]
    });
    mark(l * 20 + 2);
    stream_signal(done(c + 0, (unsigned)W), &sm.s_last);
    mark(l * 20 + 3);

    // attention (the items read q|k|v, RMSNorm and rotate q and k, append
    // k and v to the pool and attend over it)
    if (!attn_wg) ring_top_up(a, rg, wave, lane, u_lim(u + kPrO));
    uint16_t* pool_l = reinterpret_cast<uint16_t*>(a.attn.pool_layer) + (size_t)l * a.pool_layer_elems;
#ifdef QD_STEP_TRACE
    AttnArgs at = l == a.tap_layer ? a.attn_tap : a.attn;  // (trace builds) the item's
    at.trace = l == 17 ? a.trace + (size_t)wg * 1024 + 960 : nullptr;  // events of layer 17
#else
    const AttnArgs& at = l == a.tap_layer ? a.attn_tap : a.attn;
#endif
    for (int t = a_first; t < attn_n; t += W)
      attention_item<D, G, kAttnWavesPersistent, attn_pages_per_wave(1, true)>(
          at, alist, ly.q_norm, ly.k_norm, pool_l, done(c + 1, n_heads), t, in_lds,
          Waiter{a.flags + (size_t)wg * kFlagStride, phase(c + 0), a.abort_flag, a.dev_flags,
                 a.spin_limit});
    mark(l * 20 + 4);

    // O projection + residual
    {
      const StreamShare so = stream_share(a, u + kPrO, 0, W, wg);
      stream_wait(a, rg, wave, lane, phase(c + 1), u_lim(u + kPrO));
      mark(l * 20 + 5);
      if (l == a.tap_layer) {
        tap_copy(a.tap_attn, a.attn_out, a.QD);
        if (a.tap_qkv != nullptr && wg == 0)  // q|k|v: the sum of the split partials
          for (int n = tid; n < a.NQKV; n += 256) {
            const float* p = a.qkv_part + (size_t)(n / kTileRows) * a.qkv_S * kTileRows +
                             n % kTileRows;
            float v = 0.f;
            for (int s2 = 0; s2 < a.qkv_S; ++s2) v += ld_agent(p + (size_t)s2 * kTileRows);
            a.tap_qkv[n] = v;
          }
      }
      stage_input(a.attn_out, a.QD, nullptr, so.r0, so.r1);
      mark(l * 20 + 6);
      project(u + kPrO, u_lim(u + kPrO), false, resid);
      mark(l * 20 + 7);
      stream_signal(done(c + 2, (unsigned)W), &sm.s_last);
      mark(l * 20 + 8);
    }

    // gate/up + SwiGLU (rows 0-7 of a packed tile are gate channels, rows
    // 8-15 the matching up channels)
    stream_wait(a, rg, wave, lane, phase(c + 2), u_lim(u + kPrGu));
    mark(l * 20 + 9);
    if (l == a.tap_layer) tap_copy(a.tap_x_mid, a.x, a.H);
    stage_input(a.x, a.H, ly.post_norm, 0, 0);
    mark(l * 20 + 10);
    project(u + kPrGu, u_lim(u + kPrGu), true, [&](int, int rt, float y) {
      const float uv = __shfl(y, 8 + (lane & 7), 16);
      if ((lane & 15) < 8)
        st_agent(a.act + rt * 8 + (lane & 7), y / (1.f + expf(-y)) * uv);
    });
    mark(l * 20 + 11);
    stream_signal(done(c + 3, (unsigned)W), &sm.s_last);
    mark(l * 20 + 12);

    // down projection + residual
    {
      const StreamShare sd = stream_share(a, u + kPrDown, 0, W, wg);
      stream_wait(a, rg, wave, lane, phase(c + 3), u_lim(u + kPrDown));
      mark(l * 20 + 13);
      if (l == a.tap_layer) tap_copy(a.tap_act, a.act, a.I);
      stage_input(a.act, a.I, nullptr, sd.r0, sd.r1);
      mark(l * 20 + 14);
      project(u + kPrDown, u_lim(u + kPrDown), false, resid);
      mark(l * 20 + 15);
      stream_signal(done(c + 4, (unsigned)W), &sm.s_last);
      mark(l * 20 + 16);
    }
  }

  // LM head: every wave one row tile of each of the workgroup's 64-row
  // groups, all k-tiles; logits, the argmax of the workgroup's rows, then,
  // in the last workgroup to finish, of all workgroups
  const int u_lm = a.L * kUnitsPerLayer;
  stream_wait(a, rg, wave, lane, phase(cnt_index(a.L - 1, 4)), u_end);
  mark(1000);
  if (a.L - 1 == a.tap_layer) tap_copy(a.tap_x_out, a.x, a.H);
  stage_input(a.x, a.H, a.final_norm, 0, 0);
  mark(1001);
  if (a.tap_final_h != nullptr && wg == 0)  // the final RMSNorm, as the LM head applies it
    for (int i = tid; i < a.H; i += 256) a.tap_final_h[i] = ld_agent(a.x + i) * s_inv * a.final_norm[i];
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  {
    const StreamShare s = stream_share(a, u_lm, wave, W, wg);
    const unsigned short* const xin = stream_in_lane(xsh, a.H, lane);
    for (int g = s.r0; g < s.r1; ++g) {
      Acc2 acc;
      ring_mfma_run<1>(a, rg, wave, lane, u_end, s.KT, xin, acc);
      const f32x4 y = acc.total() * s_inv;
      const int row0 = (4 * g + wave) * kTileRows + (lane >> 4) * 4;
      if ((lane & 15) == 0 && a.logits != nullptr) *reinterpret_cast<f32x4*>(a.logits + row0) = y;
      float v = y[0];
      int i = row0;
#pragma unroll
      for (int q = 1; q < 4; ++q) amax_merge(v, i, y[q], row0 + q);
      wave_amax(v, i);
      amax_merge(bv, bi, v, i);
    }
  }
  mark(1002);
  if (lane == 0) { sm.amax_v[wave] = bv; sm.amax_i[wave] = bi; }
  lds_barrier();
  if (tid == 0) {
    for (int w2 = 1; w2 < 4; ++w2) amax_merge(bv, bi, sm.amax_v[w2], sm.amax_i[w2]);
    st_agent(a.amax_val + wg, bv);
    st_agent(a.amax_idx + wg, bi);
  }
  stores_done();
  lds_barrier();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.cnt + cnt_index(a.L, 0), 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.s_last = prev + 1 == (unsigned)W ? 1u : 0u;
  }
  lds_barrier();
  if (sm.s_last != 0u) {
    float v;
    int i, b;
    if (merge_amax(a.amax_val, a.amax_idx, W, 1, 1, sm.tmp, v, i, b))
      a.next_ids[0] = i == 0x7fffffff ? -1 : i;
  }

#ifdef QD_STEP_TRACE
  if (lane == 0) {
    a.trace[(size_t)wg * 1024 + 1008 + 2 * wave] = rg.t_wait;
    a.trace[(size_t)wg * 1024 + 1009 + 2 * wave] = rg.t_dot;
    a.trace[(size_t)wg * 1024 + 980 + 2 * wave] = rg.t_top;
    a.trace[(size_t)wg * 1024 + 981 + 2 * wave] = rg.t_rel;
  }
#endif
  // The last workgroup out resets the dependency counters for the next step.
  stores_done();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.exit_cnt, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (prev == (unsigned)W - 1) {
      const int n = cnt_index(a.L, 0) + 1;
      for (int i = 0; i < n; ++i) st_agent(a.cnt + i, 0u);
      for (int i = 0; i < W; ++i) st_agent(a.flags + (size_t)i * kFlagStride, 0u);
      st_agent(a.abort_flag, 0u);
      st_agent(a.exit_cnt, 0u);
    }
  }
}

}  // namespace qd
