// Prefill of prompt chunks on the matrix cores (qd_prefill_prompts).
//
// A chunk of M prompt rows runs through each layer as:
//   RMSNorm rows -> operand tiles; QKV GEMM; q/k norm + RoPE + KV append;
//   tiled causal attention -> operand tiles; O GEMM (+= residual);
//   RMSNorm rows -> operand tiles; gate/up GEMM (SwiGLU -> operand tiles);
//   down GEMM (+= residual)
// The projections are dense [M x K] . [K x N] contractions, so they run as
// GEMMs on v_mfma_f32_16x16x32_bf16: the weight tile is the A operand as
// packed, the input's bf16 hi/lo pair the B operand (two MFMAs per tile pair,
// fp32 accumulation), so the input keeps about 16 significant bits as in the
// decode kernels.  Attention is the same softmax(q.K^T/sqrt(D)).V of the
// decode step (the blog "GPU 算子与执行优化", Part 7: a prompt goes through
// the layers as one batch, causally masked, before decoding), computed per
// (segment, 16-row query block, KV head) over the paged pool with the
// blocks' K/V pages staged once in LDS for the group's query heads.
#include "qd_device.h"

namespace qd {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Two floats that are bf16 values (E4M3 values widened: exact) as a packed
// pair of bf16 bits, the first in the low half.  (The widening goes through
// v_cvt_scalef32_pk_f32_fp8: on this part it reproduces the OCP E4M3 table
// for all 256 codes, while the bf16-output form gave the first code of a
// pair for both halves in the same check.)
__device__ __forceinline__ unsigned bf_pair(f32x2 f) {
  return (__float_as_uint(f.x) >> 16) | (__float_as_uint(f.y) & 0xffff0000u);
}

// ------------------------------------------------------------------ helpers

// Segment of chunk row m (rows of segment s are [row0[s], row0[s+1])).
__device__ __forceinline__ int pf_seg_of_row(const PfSegs& sg, int m) {
  int s = 0;
  while (s + 1 < sg.n && sg.row0[s + 1] <= m) ++s;
  return s;
}

// hi/lo bf16 pairs of 4 floats, packed 2 per word.
__device__ __forceinline__ void pack_hilo4(const float* v, uint2& hi, uint2& lo) {
  unsigned h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = f2bf(v[i]);
    l[i] = f2bf(v[i] - __uint_as_float(h[i] << 16));
  }
  hi = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  lo = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
}

// ------------------------------------------------------------------ embedding

// x[m][:] = E[tokens[m]] in fp32; one wave per row, 8 columns per lane step.
__global__ __launch_bounds__(256) void pf_embed_kernel(const uint16_t* table, int V, int H,
                                                       const int* tokens, int M, float* x,
                                                       int* dev_flags) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + wave;
  if (m >= M) return;
  int tok = tokens[m];
  if (tok < 0 || tok >= V) {
    if (lane == 0) set_flag(dev_flags, QD_DEV_BAD_TOKEN);
    tok = tok < 0 ? 0 : V - 1;
  }
  const int KT = H / kTileCols, rt = tok / kTileRows, r = tok % kTileRows;
  for (int c = lane; c < H / 8; c += 64) {
    const int k0 = c * 8;
    const u32x4 w = *reinterpret_cast<const u32x4*>(
        table + ((size_t)rt * KT + k0 / kTileCols) * kTileElems + (((k0 % kTileCols) / 8) * 16 + r) * 8);
    float f[8];
    unpack8(w, f);
    f32x4* dst = reinterpret_cast<f32x4*>(x + (size_t)m * H + k0);
    dst[0] = f32x4{f[0], f[1], f[2], f[3]};
    dst[1] = f32x4{f[4], f[5], f[6], f[7]};
  }
}

// ------------------------------------------------------------------ RMSNorm rows -> operand tiles

// Row m of x [M][K] times 1/rms and the gain, as operand tiles; rows M..Mpad-1
// are written as zeros.  One wave per row.
__global__ __launch_bounds__(256) void pf_norm_kernel(const float* x, const float* gain, int K,
                                                      int M, int Mpad, float eps, uint16_t* out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + wave;
  if (m >= Mpad) return;
  const int KT = K / kTileCols;
  const float* xr = x + (size_t)m * K;
  float inv = 0.f;
  if (m < M) {
    float ss = 0.f;
    for (int c = lane; c < K / 4; c += 64) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(xr + c * 4);
      ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    ss = wave_sum(ss);
    inv = rsqrtf(ss / (float)K + eps);
  }
  for (int c = lane; c < K / 8; c += 64) {
    const int k0 = c * 8;
    float v[8];
    if (m < M) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(xr + k0);
      const f32x4 b = *reinterpret_cast<const f32x4*>(xr + k0 + 4);
      const f32x4 ga = *reinterpret_cast<const f32x4*>(gain + k0);
      const f32x4 gb = *reinterpret_cast<const f32x4*>(gain + k0 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = a[i] * inv * ga[i];
        v[4 + i] = b[i] * inv * gb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    uint2 h0, l0, h1, l1;
    pack_hilo4(v, h0, l0);
    pack_hilo4(v + 4, h1, l1);
    uint16_t* t = out + pf_tile_off(m, k0, KT);
    *reinterpret_cast<u32x4*>(t) = u32x4{h0.x, h0.y, h1.x, h1.y};
    *reinterpret_cast<u32x4*>(t + kTileElems) = u32x4{l0.x, l0.y, l1.x, l1.y};
  }
}

// ------------------------------------------------------------------ GEMM

// Y = X . W^T for one (32*WN weight rows) x (32*WM input rows) workgroup
// tile; 4 waves in 2 x 2, each 16*WN x 16*WM (WN x WM accumulators of
// 16x16).  K advances one 32-column k-tile per stage.  A stage is the
// workgroup's 2*WN weight tiles and 2*WM input tiles (hi and lo), 1 KB
// each, brought into LDS by direct global-to-LDS loads (the waves share
// them out); S stages are in flight, one workgroup per CU.  Each wave waits
// for its own loads of the next stage, then an LDS barrier makes every
// wave's tiles of that stage visible and tells that the stage just read
// into registers is free for the loads S stages ahead.  A wave reads the
// next stage's operands from LDS while its MFMAs consume the current one's
// (two register sets, alternating).
// Workgroups are laid out so that each XCD (workgroup w runs on XCD w mod 8)
// takes a contiguous range of tiles, weight block by weight block: the
// input-row blocks of one weight block run together on one XCD and the
// later ones find the weight tiles in its L2.
template <int WN, int WM>
struct PfFrag {
  bf16x8 a[WN];
  bf16x8 b[WM][2];
};

template <int MODE, int WN, int WM, int S>
__global__ __launch_bounds__(256) void pf_gemm_kernel(PfGemmArgs a) {
  constexpr int TA = 2 * WN, TB = 4 * WM, T = TA + TB;
  static_assert(T % 4 == 0, "the 4 waves share a stage's tiles evenly");
  constexpr int LPW = T / 4;
  static_assert(S >= 2 && (S - 1) * LPW <= 63, "vmcnt range");
  extern __shared__ __align__(16) unsigned char smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave & 1, wm = wave >> 1;
  const int tiles = a.nb_n * a.nb_m, per = (tiles + 7) / 8;
  const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (t >= tiles) return;
  const int nb = t / a.nb_m, mb = t % a.nb_m;
  const int KT = a.K / kTileCols, NT = a.N / kTileRows, MT = (a.M + 15) / 16;

  // this wave's loads: tiles j = wave + 4u of a stage
  const unsigned char* src[LPW];
  int step[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int j = wave + 4 * u;
    if (j < TA) {
      const int rt = min(nb * TA + j, NT - 1);
      src[u] = reinterpret_cast<const unsigned char*>(a.w + (size_t)rt * KT * kTileElems);
      step[u] = kTileElems * 2;
    } else {
      const int jb = j - TA;
      const int mt = min(mb * 2 * WM + (jb >> 1), MT - 1);
      src[u] = reinterpret_cast<const unsigned char*>(a.x + ((size_t)mt * KT * 2 + (jb & 1)) *
                                                                kTileElems);
      step[u] = kTileElems * 4;
    }
  }
  auto issue = [&](int kt, int slot) {
#pragma unroll
    for (int u = 0; u < LPW; ++u)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const u32x4*>(src[u] + (size_t)kt * step[u]) + lane,
          smem + ((size_t)slot * T + wave + 4 * u) * 1024, 16, 0, 0);
  };
  auto read_frag = [&](PfFrag<WN, WM>& f, int slot) {
    const unsigned char* st = smem + (size_t)slot * T * 1024 + lane * 16;
#pragma unroll
    for (int i = 0; i < WN; ++i)
      f.a[i] = *reinterpret_cast<const bf16x8*>(st + (wn * WN + i) * 1024);
#pragma unroll
    for (int j = 0; j < WM; ++j)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
        f.b[j][hl] = *reinterpret_cast<const bf16x8*>(st + (TA + (wm * WM + j) * 2 + hl) * 1024);
  };

  f32x4 acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const PfFrag<WN, WM>& f) {
#pragma unroll
    for (int hl = 0; hl < 2; ++hl)
#pragma unroll
      for (int j = 0; j < WM; ++j)
#pragma unroll
        for (int i = 0; i < WN; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j][hl], acc[i][j], 0, 0, 0);
  };
  // one k-tile kt < KT-1: make stage kt+1 visible, refill the slot of stage
  // kt (already read into cur) with stage kt+S, read stage kt+1 into nxt,
  // multiply cur.  (The last k-tile only multiplies: no branch inside the
  // loop body, so the compiler sees that cur's LDS reads have completed.)
  auto step_k = [&](int kt, const PfFrag<WN, WM>& cur, PfFrag<WN, WM>& nxt) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (kt + S - 1 <= KT - 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * LPW));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    if (kt + S < KT) issue(kt + S, kt % S);
    read_frag(nxt, (kt + 1) % S);
    mma(cur);
  };

#pragma unroll
  for (int s = 0; s < S; ++s)
    if (s < KT) issue(s, s);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (KT >= S)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 1) * LPW));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  PfFrag<WN, WM> f0, f1;
  read_frag(f0, 0);
  int kt = 0;
  for (; kt + 2 < KT; kt += 2) {
    step_k(kt, f0, f1);
    step_k(kt + 1, f1, f0);
  }
  if (kt + 2 == KT) {
    step_k(kt, f0, f1);
    mma(f1);
  } else {
    mma(f0);
  }

  // epilogue: acc[i][j] lane l holds rows 4*(l/16)..+3 of weight row tile
  // rt, input row m = 16*(m tile) + l%16
  const int r0 = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < WN; ++i) {
    const int rt = nb * TA + wn * WN + i;
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      const int m = (mb * 2 * WM + wm * WM + j) * 16 + (lane & 15);
      const bool ok = rt < NT && m < a.M;
      if constexpr (MODE == kPfSwiGLU) {
        // rows 0-7 of a packed tile are gate rows 8rt.., rows 8-15 the up
        // rows of the same channels: lanes l and l+32 hold a channel's pair
        f32x4 up;
#pragma unroll
        for (int r = 0; r < 4; ++r) up[r] = __shfl_xor(acc[i][j][r], 32);
        if (ok && lane < 32) {
          const int c0 = rt * 8 + r0;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float g = acc[i][j][r];
            v[r] = g / (1.f + expf(-g)) * up[r];
          }
          uint2 hi, lo;
          pack_hilo4(v, hi, lo);
          uint16_t* dst = a.act + pf_tile_off(m, c0, a.N / 2 / kTileCols);
          *reinterpret_cast<uint2*>(dst) = hi;
          *reinterpret_cast<uint2*>(dst + kTileElems) = lo;
        }
      } else if (ok) {
        f32x4* dst = reinterpret_cast<f32x4*>(a.out + (size_t)m * a.ldo + rt * 16 + r0);
        if constexpr (MODE == kPfResid)
          *dst = *dst + acc[i][j];
        else
          *dst = acc[i][j];
      }
    }
  }
}

// ------------------------------------------------------------------ q/k norm, RoPE, KV append

// One wave per (row, head) of q heads then KV heads; lane i < D/2 holds
// elements i and i + D/2 (the NeoX rotation pairs).  q heads: RMSNorm with
// the q gain, RoPE at the row's position, times the softmax scale (and, for
// an 8-bit pool, K's scale: attention multiplies q by K's codes), stored as a
// bf16 pair.  KV heads: k as q with the k gain (no scale) and v as is, both
// rounded to the pool's element (bf16, or E4M3 of value / scale) into the
// row's slot of the pool.
template <int D, class KV>
__global__ __launch_bounds__(256) void pf_qk_kernel(PfAttnArgs a) {
  using Elem = typename KV::Elem;
  constexpr int HALF = D / 2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int NH = a.Hq + a.Hkv;
  const int task = blockIdx.x * 4 + wave;
  if (task >= a.M * NH) return;
  const int m = task / NH, hh = task % NH;
  const int s = pf_seg_of_row(a.seg, m);
  const int p = a.seg.pos0[s] + m - a.seg.row0[s];
  const bool act = lane < HALF;
  const int i = act ? lane : 0;
  const int QD = a.Hq * D, KD = a.Hkv * D;
  const float* row = a.qkv + (size_t)m * (QD + 2 * KD);
  const int off = hh < a.Hq ? hh * D : QD + (hh - a.Hq) * D;
  float x1 = act ? row[off + i] : 0.f, x2 = act ? row[off + i + HALF] : 0.f;
  const float* gn = hh < a.Hq ? a.q_gain : a.k_gain;
  const float inv = rsqrtf(wave_sum(x1 * x1 + x2 * x2) / (float)D + a.eps);
  const float y1 = x1 * inv * gn[i], y2 = x2 * inv * gn[i + HALF];
  const float cs = a.rope_cos[(size_t)p * HALF + i], sn = a.rope_sin[(size_t)p * HALF + i];
  const float r1 = y1 * cs - y2 * sn, r2 = y2 * cs + y1 * sn;
  if (hh < a.Hq) {
    if (act) {
      const size_t q = ((size_t)m * a.Hq + hh) * D + i;
      const float qs = KV::kFp8 ? a.scale * a.k_scale : a.scale;
      const float v1 = r1 * qs, v2 = r2 * qs;
      const unsigned h1 = f2bf(v1), h2 = f2bf(v2);
      a.q_hi[q] = (uint16_t)h1;
      a.q_hi[q + HALF] = (uint16_t)h2;
      a.q_lo[q] = (uint16_t)f2bf(v1 - __uint_as_float(h1 << 16));
      a.q_lo[q + HALF] = (uint16_t)f2bf(v2 - __uint_as_float(h2 << 16));
    }
    return;
  }
  const int g = hh - a.Hq;
  int page = a.block_tables[(size_t)s * a.max_pages + p / kPage];
  if (page < 0 || page >= a.num_pages) {
    if (lane == 0) set_flag(a.dev_flags, QD_DEV_BAD_PAGE);
    page = page < 0 ? 0 : a.num_pages - 1;
  }
  if (!act) return;
  Elem* kd = reinterpret_cast<Elem*>(a.pool_layer) +
             (((size_t)page * 2 + 0) * a.Hkv + g) * kPage * D + (p % kPage) * D;
  Elem* vd = kd + (size_t)a.Hkv * kPage * D;
  kd[i] = KV::encode(r1, a.k_inv);
  kd[i + HALF] = KV::encode(r2, a.k_inv);
  const float* vr = row + QD + KD + g * D;
  vd[i] = KV::encode(vr[i], a.v_inv);
  vd[i + HALF] = KV::encode(vr[i + HALF], a.v_inv);
}

// ------------------------------------------------------------------ tiled causal attention

// One workgroup per (segment, 16-row query block, KV head); wave w takes
// query head g*G + w.  For each page of the block's context (positions
// 0 .. the block's last), the workgroup stages the page's K and V in LDS
// with direct global-to-LDS loads, kNs pages in flight.  K of a bf16 pool
// lands as 1 KB A-operand tiles (lane l: key l%16, head dims 32*kk +
// 8*(l/16)..+7); K of an 8-bit pool lands row-major and each lane widens its
// 8 codes to bf16 (exact: every E4M3 value is a bf16 value).  V lands
// row-major, each 1 KB chunk padded by 64 bytes so that the transposed reads
// below spread over the banks.  Per page a wave forms S^T = K . Q^T (16 keys
// x 16 queries) with 16x16x32 MFMAs on q's hi and lo (q carries the softmax
// scale, and K's scale for an 8-bit pool), masks keys past each query's
// position, updates each query's running maximum and sum (online softmax, as
// the decode kernels), and accumulates O^T += V^T . P^T with 16x16x16 MFMAs
// on P's hi and lo.  Lane l ends with O^T[d = 16*dt + 4*(l/16)..+3][query
// l%16] (times V's scale for an 8-bit pool) and writes the block's rows as
// operand tiles for the O projection.
template <int D, int G, class KV>
__global__ __launch_bounds__(64 * G) void pf_attn_kernel(PfAttnArgs a) {
  constexpr int EB = KV::kFp8 ? 1 : 2;       // bytes per pool element
  constexpr int KK = D / 32;                 // 32-dim steps of q.k
  constexpr int PB = kPage * D * EB;         // bytes of one page's K (or V) of one head
  constexpr int KCH = PB / 1024;             // 1 KB chunks of K, and of V
  constexpr int KPC = 1024 / (D * EB);       // keys per V chunk
  constexpr int VSTRIDE = 1024 + 64;         // padded V chunk
  constexpr int SLOT = KCH * 1024 + KCH * VSTRIDE;
  constexpr int CH = 2 * KCH;                // 1 KB loads per page
  constexpr int LPW = (CH + G - 1) / G;      // ... per wave (fewer for the last waves if
                                             // CH is not a multiple of G)
  constexpr int kNs = 4;
  static_assert((kNs - 2) * LPW <= 63, "vmcnt range");
  constexpr int DT = D / 16;
  __shared__ __align__(16) unsigned char lds[kNs * SLOT];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.x % a.Hkv;
  const int nqb = a.seg.qb0[a.seg.n];
  const int item = nqb - 1 - (int)(blockIdx.x / a.Hkv);  // longest blocks first
  int s = 0;
  while (s + 1 < a.seg.n && a.seg.qb0[s + 1] <= item) ++s;
  const int qb = item - a.seg.qb0[s];
  const int r_begin = a.seg.row0[s] + 16 * qb;
  const int nrows = min(16, a.seg.row0[s + 1] - r_begin);
  const int p_first = a.seg.pos0[s] + 16 * qb;
  const int npages = (p_first + nrows - 1) / kPage + 1;
  const int h = g * G + wave;
  const int* table = a.block_tables + (size_t)s * a.max_pages;
  // this wave's loads per page are chunks c = wave + G*u < CH; a wave with
  // fewer than LPW of them waits for all of its loads
  const bool full_share = (wave + G * (LPW - 1)) < CH;

  // q^T fragments (B operand): lane l holds query l%16, dims 32*kk + 8*(l/16)..+7
  const int qr = r_begin + min(lane & 15, nrows - 1);
  bf16x8 qf[KK][2];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const size_t o = ((size_t)qr * a.Hq + h) * D + 32 * kk + 8 * (lane >> 4);
    qf[kk][0] = *reinterpret_cast<const bf16x8*>(a.q_hi + o);
    qf[kk][1] = *reinterpret_cast<const bf16x8*>(a.q_lo + o);
  }

  // the item's page ids 64 at a time in a register (lane l: page 64c + l of
  // chunk c), so that finding a page in the loop needs no memory round trip
  // (a load there would have to wait for every K/V load in flight)
  int tab_chunk = 0;
  int tab_reg = lane < npages ? table[lane] : 0;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // q fragments and page ids in registers
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  auto issue = [&](int pg, int slot) {
    if ((pg >> 6) != tab_chunk) {
      tab_chunk = pg >> 6;
      const int i = 64 * tab_chunk + lane;
      tab_reg = i < npages ? table[i] : 0;
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // once per 64 pages
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    int page = __builtin_amdgcn_readlane(tab_reg, pg & 63);
    if (page < 0 || page >= a.num_pages) {
      if (lane == 0) set_flag(a.dev_flags, QD_DEV_BAD_PAGE);
      page = page < 0 ? 0 : a.num_pages - 1;
    }
    const unsigned char* kb = a.pool_layer + (((size_t)page * 2 + 0) * a.Hkv + g) * PB;
    const unsigned char* vb = kb + (size_t)a.Hkv * PB;
    unsigned char* base = lds + (size_t)slot * SLOT;
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int c = wave + G * u;
      if (c >= CH) break;  // wave-uniform
      if (c < KCH) {
        const unsigned char* gp =
            KV::kFp8 ? kb + c * 1024 + lane * 16
                     : kb + ((lane & 15) * D + 32 * c + 8 * (lane >> 4)) * 2;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4*>(gp), base + c * 1024, 16,
                                         0, 0);
      } else {
        const int v = c - KCH;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4*>(vb + v * 1024 + lane * 16),
                                         base + KCH * 1024 + v * VSTRIDE, 16, 0, 0);
      }
    }
  };
  // this lane's K A-operand for dims 32*kk.. of the staged page
  auto k_frag = [&](const unsigned char* base, int kk) -> bf16x8 {
    if constexpr (KV::kFp8) {
      const u32x2 c = *reinterpret_cast<const u32x2*>(base + (lane & 15) * D + 32 * kk +
                                                      8 * (lane >> 4));
      const f32x2 f[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.x, 1.0f, false),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.x, 1.0f, true),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.y, 1.0f, false),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.y, 1.0f, true)};
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = bf_pair(f[i]);
      return __builtin_bit_cast(bf16x8, w);
    } else {
      return *reinterpret_cast<const bf16x8*>(base + kk * 1024 + lane * 16);
    }
  };
  // V^T A operand: lane l holds dim `dim` of keys 4*(l/16)..+3 as bf16
  auto v_frag = [&](const unsigned char* base, int dim) -> s16x4 {
    auto at = [&](int key) {
      return base + KCH * 1024 + (key / KPC) * VSTRIDE + (key % KPC) * D * EB + dim * EB;
    };
    const int k0 = 4 * (lane >> 4);
    s16x4 va;
    if constexpr (KV::kFp8) {
      const unsigned w = (unsigned)*at(k0) | ((unsigned)*at(k0 + 1) << 8) |
                         ((unsigned)*at(k0 + 2) << 16) | ((unsigned)*at(k0 + 3) << 24);
      const u32x2 pr = u32x2{bf_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false)),
                             bf_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true))};
      va = __builtin_bit_cast(s16x4, pr);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) va[r] = *reinterpret_cast<const short*>(at(k0 + r));
    }
    return va;
  };

  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int qpos = p_first + (lane & 15);
  const bool qvalid = (lane & 15) < nrows;

#pragma unroll
  for (int st = 0; st < kNs - 1; ++st)
    if (st < npages) issue(st, st);
  for (int pg = 0; pg < npages; ++pg) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (full_share && pg + kNs - 2 < npages)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((kNs - 2) * LPW));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    if (pg + kNs - 1 < npages) issue(pg + kNs - 1, (pg + kNs - 1) % kNs);
    const unsigned char* base = lds + (size_t)(pg % kNs) * SLOT;
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 ka = k_frag(base, kk);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[kk][0], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[kk][1], s1, 0, 0, 0);
    }
    // lane l: keys 4*(l/16)+r of the page, query l%16
    float sc[4], mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kp = pg * kPage + 4 * (lane >> 4) + r;
      sc[r] = (qvalid && kp <= qpos) ? s0[r] + s1[r] : -INFINITY;
      mx = fmaxf(mx, sc[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
    float p[4], ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = (sc[r] == -INFINITY) ? 0.f : expf(sc[r] - m_new);
      ps += p[r];
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    s16x4 ph, pl;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const unsigned hb = f2bf(p[r]);
      ph[r] = (short)hb;
      pl[r] = (short)f2bf(p[r] - __uint_as_float(hb << 16));
    }
    // V^T A operand: lane l holds dim 16*dt + l%16 of keys 4*(l/16)..+3
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const s16x4 va = v_frag(base, 16 * dt + (lane & 15));
      o[dt] = o[dt] * alpha;
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph, o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl, o[dt], 0, 0, 0);
    }
  }

  if (qvalid) {
    const float inv = (KV::kFp8 ? a.v_scale : 1.f) / l_run;
    const int m = r_begin + (lane & 15);
    const int KT = a.Hq * D / kTileCols;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = o[dt][r] * inv;
      uint2 hi, lo;
      pack_hilo4(v, hi, lo);
      uint16_t* dst = a.out + pf_tile_off(m, h * D + dt * 16 + 4 * (lane >> 4), KT);
      *reinterpret_cast<uint2*>(dst) = hi;
      *reinterpret_cast<uint2*>(dst + kTileElems) = lo;
    }
  }
}

// ------------------------------------------------------------------ LM head rows

// The last row of segments 0..n-1 into the decode step's buffers, as the
// embedding launch leaves them: x [b][H], partial sums of squares
// [H/16][Bmax] and (MFMA consumers) the bf16 pairs of x times the final gain.
__global__ __launch_bounds__(256) void pf_head_rows_kernel(const float* x, int H, PfSegs seg,
                                                           const float* gain, float* x_out,
                                                           float* ssq_out, int Bmax,
                                                           uint16_t* xo_hi, uint16_t* xo_lo) {
  const int b = blockIdx.x;
  const int r = seg.row0[b + 1] - 1;
  for (int k = threadIdx.x; k < H; k += 256) {
    const float xv = x[(size_t)r * H + k];
    x_out[(size_t)b * H + k] = xv;
    if (xo_hi != nullptr) {
      const float v = xv * gain[k];
      const unsigned hb = f2bf(v);
      xo_hi[(size_t)b * H + k] = (uint16_t)hb;
      xo_lo[(size_t)b * H + k] = (uint16_t)f2bf(v - __uint_as_float(hb << 16));
    }
    const float ss = group_sum(xv * xv, kSsqRows);
    if (k % kSsqRows == 0) ssq_out[(size_t)(k / kSsqRows) * Bmax + b] = ss;
  }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_pf_embed(const uint16_t* table, int V, int H, const int* tokens, int M,
                           float* x, int* dev_flags, hipStream_t s) {
  hipLaunchKernelGGL(pf_embed_kernel, dim3((M + 3) / 4), dim3(256), 0, s, table, V, H, tokens, M,
                     x, dev_flags);
  return hipGetLastError();
}

hipError_t launch_pf_norm(const float* x, const float* gain, int K, int M, int Mpad, float eps,
                          uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(pf_norm_kernel, dim3((Mpad + 3) / 4), dim3(256), 0, s, x, gain, K, M, Mpad,
                     eps, out);
  return hipGetLastError();
}

// Stages of a GEMM workgroup: as many as 72 KB of LDS hold (two workgroups
// per CU), within the vmcnt range.
constexpr int pf_stages(int WN, int WM) {
  const int T = 2 * WN + 4 * WM, lpw = T / 4;
  const int by_lds = 72 / T, by_cnt = 63 / lpw + 1;
  return by_lds < by_cnt ? by_lds : by_cnt;
}

template <int MODE, int WN, int WM>
static hipError_t launch_pf_gemm_t(const PfGemmArgs& a, hipStream_t s) {
  constexpr int kStages = pf_stages(WN, WM);
  constexpr size_t lds = (size_t)kStages * (2 * WN + 4 * WM) * 1024;
  static bool attr_set = false;
  const void* fn = reinterpret_cast<const void*>(&pf_gemm_kernel<MODE, WN, WM, kStages>);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int tiles = a.nb_n * a.nb_m;
  hipLaunchKernelGGL((pf_gemm_kernel<MODE, WN, WM, kStages>), dim3(8 * ((tiles + 7) / 8)),
                     dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_pf_gemm_m(const PfGemmArgs& a, int wn, int wm, hipStream_t s) {
  if (wn == 4 && wm == 4) return launch_pf_gemm_t<MODE, 4, 4>(a, s);
  if (wn == 2 && wm == 4) return launch_pf_gemm_t<MODE, 2, 4>(a, s);
  if (wn == 4 && wm == 2) return launch_pf_gemm_t<MODE, 4, 2>(a, s);
  if (wn == 2 && wm == 2) return launch_pf_gemm_t<MODE, 2, 2>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_pf_gemm(const PfGemmArgs& a, int mode, int wn, int wm, hipStream_t s) {
  switch (mode) {
    case kPfStore: return launch_pf_gemm_m<kPfStore>(a, wn, wm, s);
    case kPfResid: return launch_pf_gemm_m<kPfResid>(a, wn, wm, s);
    case kPfSwiGLU: return launch_pf_gemm_m<kPfSwiGLU>(a, wn, wm, s);
    default: return hipErrorInvalidValue;
  }
}

template <class KV>
static hipError_t launch_pf_qk_t(const PfAttnArgs& a, int head_dim, hipStream_t s) {
  const long long tasks = (long long)a.M * (a.Hq + a.Hkv);
  const dim3 grid((unsigned)((tasks + 3) / 4));
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((pf_qk_kernel<64, KV>), grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL((pf_qk_kernel<128, KV>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pf_qk(const PfAttnArgs& a, int head_dim, hipStream_t s) {
  return a.kv_fp8 ? launch_pf_qk_t<KvFp8>(a, head_dim, s) : launch_pf_qk_t<KvBf16>(a, head_dim, s);
}

template <int D, int G, class KV>
static hipError_t launch_pf_attn_t(const PfAttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.seg.qb0[a.seg.n] * a.Hkv));
  hipLaunchKernelGGL((pf_attn_kernel<D, G, KV>), grid, dim3(64 * G), 0, s, a);
  return hipGetLastError();
}

template <class KV>
static hipError_t launch_pf_attn_kv(const PfAttnArgs& a, int head_dim, int group, hipStream_t s) {
  if (head_dim == 128 && group == 4) return launch_pf_attn_t<128, 4, KV>(a, s);
  if (head_dim == 128 && group == 2) return launch_pf_attn_t<128, 2, KV>(a, s);
  if (head_dim == 128 && group == 1) return launch_pf_attn_t<128, 1, KV>(a, s);
  if (head_dim == 64 && group == 4) return launch_pf_attn_t<64, 4, KV>(a, s);
  if (head_dim == 64 && group == 2) return launch_pf_attn_t<64, 2, KV>(a, s);
  if (head_dim == 64 && group == 1) return launch_pf_attn_t<64, 1, KV>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_pf_attn(const PfAttnArgs& a, int head_dim, int group, hipStream_t s) {
  return a.kv_fp8 ? launch_pf_attn_kv<KvFp8>(a, head_dim, group, s)
                  : launch_pf_attn_kv<KvBf16>(a, head_dim, group, s);
}

hipError_t launch_pf_head_rows(const float* x, int H, const PfSegs& seg, int n, const float* gain,
                               float* x_out, float* ssq_out, int Bmax, uint16_t* xo_hi,
                               uint16_t* xo_lo, hipStream_t s) {
  hipLaunchKernelGGL(pf_head_rows_kernel, dim3(n), dim3(256), 0, s, x, H, seg, gain, x_out,
                     ssq_out, Bmax, xo_hi, xo_lo);
  return hipGetLastError();
}

}  // namespace qd
