// The persistent decode-step kernel (one cooperative launch per step).
// Included once per batch-column count by the qd_step_nb*.hip translation
// units, which instantiate it, so that the large kernels compile in parallel.
#pragma once

#include "qd_device.h"

namespace qd {

// Weight tiles a wave keeps in flight inside the persistent kernel.
constexpr int kPersistentTiles = kMaxTilesInFlight;

#ifdef QD_STEP_TRACE
// A wait that also records when it was satisfied (trace builds only).
struct TracedWaiter {
  static constexpr bool kInLaunch = true;
  Waiter w;
  unsigned long long* t;
  __device__ void operator()() const {
    w();
    if (threadIdx.x == 0) *t = __builtin_amdgcn_s_memrealtime();
  }
};
#endif

__device__ __forceinline__ int gemv_row_groups(const GemvArgs& g) {
  return g.N / (kTileRows * g.rt);
}
__device__ __forceinline__ int gemv_items(const GemvArgs& g) { return gemv_row_groups(g) * g.S; }

// The whole decode step in one cooperative launch.  Items are numbered in
// step order (embedding, then per layer QKV, attention, O, gate/up, down,
// then the LM head) and workgroup w takes items w, w + grid, w + 2*grid, ...
// Each stage waits only on counters of earlier stages, and a workgroup takes
// its items in step order, so the step always makes progress when every
// workgroup is resident (the cooperative launch guarantees it).
template <int NB, int D, int G>
__global__ __launch_bounds__(256) void step_kernel(const StepArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const long nwg = gridDim.x, wg = blockIdx.x;
  long base = 0;
#ifdef QD_STEP_TRACE
  // (phase, start, wait satisfied, end) of every item this workgroup runs,
  // 100 MHz clock
  __shared__ unsigned long long t_wait;
  int trace_phase = 0, nrec = 0;
  unsigned long long* tr = a.trace + (size_t)wg * 1024 * 4;
  auto for_items = [&](int n, auto&& fn) {
    const long first = base + ((wg - base) % nwg + nwg) % nwg;
    for (long j = first; j < base + n; j += nwg) {
      const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
      if (threadIdx.x == 0) t_wait = t0;
      fn((int)(j - base));
      const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
      if (threadIdx.x == 0 && nrec < 1024) {
        tr[nrec * 4 + 0] = (unsigned long long)trace_phase;
        tr[nrec * 4 + 1] = t0;
        tr[nrec * 4 + 2] = t_wait;
        tr[nrec * 4 + 3] = t1;
      }
      ++nrec;
    }
    base += n;
    ++trace_phase;
  };
  auto waiter = [&](unsigned phase) {
    return TracedWaiter{Waiter{a.flags + (size_t)wg * kFlagStride, phase, a.abort_flag,
                               a.dev_flags, a.spin_limit}, &t_wait};
  };
#else
  auto for_items = [&](int n, auto&& fn) {
    const long first = base + ((wg - base) % nwg + nwg) % nwg;
    for (long j = first; j < base + n; j += nwg) fn((int)(j - base));
    base += n;
  };
  auto waiter = [&](unsigned phase) {
    return Waiter{a.flags + (size_t)wg * kFlagStride, phase, a.abort_flag, a.dev_flags,
                  a.spin_limit};
  };
#endif
  const unsigned rg_o = (unsigned)gemv_row_groups(a.o);
  const unsigned rg_down = (unsigned)gemv_row_groups(a.down);
  // QKV leaves split partials that attention sums: that stage is complete
  // when every item is
  const unsigned n_qkv = (unsigned)gemv_items(a.qkv);
  const unsigned rg_gu = (unsigned)gemv_row_groups(a.gu);
  const unsigned n_heads = (unsigned)(a.attn.B * a.attn.Hkv);
  // the attention work list (positions are inputs of the step)
  const AttnList alist = attn_list<attn_pages_per_split(1, true)>(a.attn);
  const int attn_n = attn_items(alist, a.attn.B);
  // stage with counter index i completes phase i + 1 (0: nothing done yet)
  auto done = [&](int i, unsigned target) {
    return Done{a.cnt + i, target, (unsigned)i + 1u, a.flags, (int)nwg};
  };
  auto phase = [](int i) { return (unsigned)i + 1u; };

  for_items(a.embed.B, [&](int b) {
    __syncthreads();
    embed_item(a.embed, done(kCntEmbed, (unsigned)a.embed.B), b);
  });

  for (int l = 0; l < a.L; ++l) {
    const LayerDev ly = a.layers[l];
    const int c = cnt_index(l, 0);
    const unsigned x_ready = l == 0 ? phase(kCntEmbed) : phase(cnt_index(l - 1, 4));

    for_items(gemv_items(a.qkv), [&](int it) {
      gemv_item<NB, kPartial, kPersistentTiles>(a.qkv, ly.qkv, ly.in_norm, done(c + 0, n_qkv),
                                                it, smem, waiter(x_ready));
    });
    uint16_t* pool_l = a.attn.pool_layer + (size_t)l * a.pool_layer_elems;
    for_items(attn_n, [&](int it) {
      attention_item<D, G, kAttnWavesPersistent, attn_pages_per_wave(1, true)>(
          a.attn, alist, ly.q_norm, ly.k_norm, pool_l, done(c + 1, n_heads), it, smem,
          waiter(phase(c + 0)));
    });
    for_items(gemv_items(a.o), [&](int it) {
      gemv_item<NB, kResid, kPersistentTiles>(a.o, ly.o, nullptr, done(c + 2, rg_o), it, smem,
                                              waiter(phase(c + 1)));
    });
    for_items(gemv_items(a.gu), [&](int it) {
      gemv_item<NB, kSwiGLU, kPersistentTiles>(a.gu, ly.gu, ly.post_norm, done(c + 3, rg_gu),
                                               it, smem, waiter(phase(c + 2)));
    });
    for_items(gemv_items(a.down), [&](int it) {
      gemv_item<NB, kResid, kPersistentTiles>(a.down, ly.down, nullptr, done(c + 4, rg_down),
                                              it, smem, waiter(phase(c + 3)));
    });
  }

  for_items(gemv_items(a.lm), [&](int it) {
    gemv_item<NB, kArgmax, kPersistentTiles>(a.lm, a.lm.w, a.lm.gain, no_done(), it, smem,
                                             waiter(phase(cnt_index(a.L - 1, 4))));
  });

  // The last workgroup out resets the dependency counters for the next step.
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.exit_cnt, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (prev == (unsigned)nwg - 1) {
      const int n = 1 + a.L * kCntPerLayer;
      for (int i = 0; i < n; ++i) st_agent(a.cnt + i, 0u);
      for (long i = 0; i < nwg; ++i) st_agent(a.flags + (size_t)i * kFlagStride, 0u);
      st_agent(a.abort_flag, 0u);
      st_agent(a.exit_cnt, 0u);
    }
  }
}


template <int NB>
hipError_t step_dispatch(int head_dim, int group, const StepArgs* a, int grid, size_t lds,
                         hipStream_t s, int* max_grid, int num_cus) {
  const void* fn = nullptr;
  if (head_dim == 128 && group == 4) fn = reinterpret_cast<const void*>(&step_kernel<NB, 128, 4>);
  if (head_dim == 64 && group == 2) fn = reinterpret_cast<const void*>(&step_kernel<NB, 64, 2>);
  if (fn == nullptr) return hipErrorInvalidValue;
  if (max_grid != nullptr) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds);
    if (e != hipSuccess) return e;
    *max_grid = per_cu * num_cus;
    return hipSuccess;
  }
  void* args[] = {const_cast<StepArgs*>(a)};
  return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(256), args, (unsigned)lds, s);
}

}  // namespace qd
