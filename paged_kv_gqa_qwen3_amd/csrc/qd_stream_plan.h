// Which weight tiles each wave of the batch-1 streaming step kernel loads,
// in which order, and the bookkeeping of its ring of LDS slots.  Host and
// device code: the kernel (qd_stream.h) issues the loads; a CPU check
// replays every wave of every workgroup to show that each load stays inside
// its matrix and that the tiles arrive in the order they are consumed.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "qd_internal.h"

#if defined(__HIPCC__)
#define QD_HD __host__ __device__ __forceinline__
#else
#define QD_HD inline
#endif

namespace qd {

// Tiles are consumed in batches of up to kBatch: one wait, then the batch's
// LDS reads issued together, so that a wave (alone on its SIMD) exposes one
// LDS round trip per batch instead of one per tile.
constexpr int kBatch = 4;

// The step's weight stream is a sequence of units: 4 projections per layer
// (QKV, O, gate/up, down) in layer order, then the LM head; u_end (=
// 4*L + 1) marks its end.
constexpr int kUnitsPerLayer = 4;
// A projection's k-tiles are dealt round robin to the workgroup's 4 waves.
constexpr int kStreamKStep = 4;
enum StreamProj : int { kPrQkv = 0, kPrO = 1, kPrGu = 2, kPrDown = 3 };

QD_HD int stream_u_end(const StreamArgs& a) { return a.L * kUnitsPerLayer + 1; }

// One wave's share of one unit.  A unit of R row tiles (the LM head: 64-row
// groups) with S K-splits has R*S pieces, piece r being k-tiles
// [(r%S)*kps, min(KT, (r%S+1)*kps)) of row tile r/S; the workgroup owns
// pieces [r0, r1), and of each the wave takes k-tiles kb + kstart, kb +
// kstart + kstep, ... (the LM head: row tile 4*g + wave of group g, every
// k-tile).
struct StreamShare {
  const uint16_t* w;
  int KT, R, S, kps, r0, r1, kstart, kstep;
  bool lm;
};

// Workgroups are dealt to the chip's 8 XCDs round robin (wg % 8); a
// workgroup's place in every partition is its index in XCD-major order, so
// that each XCD gets a balanced share of every unit.
QD_HD int stream_place(int wg, int W) { return W % 8 == 0 ? (wg % 8) * (W / 8) + wg / 8 : wg; }

// Workgroup wg of W owns pieces [q*P/W, (q+1)*P/W) of a unit with P
// pieces, q = stream_place(wg, W).
QD_HD StreamShare stream_share(const StreamArgs& a, int u, int wave, int W, int wg) {
  StreamShare s;
  if (u >= a.L * kUnitsPerLayer) {
    s.w = a.lm; s.KT = a.H / kTileCols; s.R = a.V / kRowsPerGroup; s.S = 1;
    s.kstart = 0; s.kstep = 1; s.lm = true;
  } else {
    const int p = u % kUnitsPerLayer;
    s.w = a.w[u];
    s.KT = (p == kPrO ? a.QD : p == kPrDown ? a.I : a.H) / kTileCols;
    s.R = (p == kPrQkv ? a.NQKV : p == kPrGu ? 2 * a.I : a.H) / kTileRows;
    s.S = p == kPrQkv ? a.qkv_S : 1;
    s.kstart = wave; s.kstep = kStreamKStep; s.lm = false;
  }
  s.kps = (s.KT + s.S - 1) / s.S;
  const unsigned P = (unsigned)s.R * (unsigned)s.S;
  const unsigned q = (unsigned)stream_place(wg, W);
  s.r0 = (int)(q * P / (unsigned)W);
  s.r1 = (int)((q + 1) * P / (unsigned)W);
  return s;
}

// k-tile range [kb, ke) of piece r.
QD_HD void stream_piece(const StreamShare& s, int r, int& kb, int& ke) {
  kb = (r % s.S) * s.kps;
  ke = kb + s.kps < s.KT ? kb + s.kps : s.KT;
}

// k-tiles of piece r that the wave takes.
QD_HD int stream_piece_tiles(const StreamShare& s, int r) {
  int kb, ke;
  stream_piece(s, r, kb, ke);
  return kb + s.kstart < ke ? (ke - kb - s.kstart + s.kstep - 1) / s.kstep : 0;
}

QD_HD const unsigned char* stream_tile(const StreamShare& s, int r, int k, int wave) {
  const int rt = s.lm ? 4 * r + wave : r / s.S;
  return reinterpret_cast<const unsigned char*>(s.w) + ((size_t)rt * s.KT + k) * 1024;
}

// One run of a wave's tile stream: n tiles at p, p + stride, ... (bytes),
// all of unit u.  The host lists each wave's runs in stream order
// (stream_runs), ending with a run of no tiles in unit u_end; the kernel's
// loader walks them with scalar loads, so that its state stays small.
struct StreamRun {
  const unsigned char* p;
  uint32_t n_u;     // n | u << 16
  uint32_t stride;
};
static_assert(sizeof(StreamRun) == 16, "16-byte runs");

// Host: emit(p, n, stride, u) for the runs of wave `wave` of workgroup wg,
// in stream order, then the terminating run.
template <class Emit>
inline void stream_runs(const StreamArgs& a, int W, int wg, int wave, const Emit& emit) {
  const int u_end = stream_u_end(a);
  for (int u = 0; u < u_end; ++u) {
    const StreamShare s = stream_share(a, u, wave, W, wg);
    for (int r = s.r0; r < s.r1; ++r) {
      int kb, ke;
      stream_piece(s, r, kb, ke);
      const int n = stream_piece_tiles(s, r);
      if (n > 0) emit(stream_tile(s, r, kb + s.kstart, wave), n, s.kstep * 1024, u);
    }
  }
  emit(static_cast<const unsigned char*>(nullptr), 0, 0, u_end);
}

// The loader: the current run, the next tile of it and the tiles left in
// it, and the ring counts (tiles issued and consumed so far, the slot the
// next load goes to).
struct StreamLoader {
  const StreamRun* run;
  const unsigned char* p;
  int n, u, stride;
  int issued, consumed, slot;
};

QD_HD void stream_fetch(StreamLoader& c) {
#if defined(__HIP_DEVICE_COMPILE__)
  // constant address space: read with scalar loads (the runs never change)
  const __attribute__((address_space(4))) StreamRun* r =
      (const __attribute__((address_space(4))) StreamRun*)c.run;
  c.p = r->p;
  const uint32_t nu = r->n_u;
  c.stride = (int)r->stride;
#else
  c.p = c.run->p;
  const uint32_t nu = c.run->n_u;
  c.stride = (int)c.run->stride;
#endif
  c.n = (int)(nu & 0xffffu);
  c.u = (int)(nu >> 16);
}

QD_HD void stream_start(StreamLoader& c, const StreamRun* runs) {
  c.run = runs;
  c.issued = c.consumed = c.slot = 0;
  stream_fetch(c);
}

// Issue loads (issue(tile, slot)) until kStreamRing tiles are loaded or in
// flight ahead of the consumer, but none of a unit after u_limit and none
// past the end of the stream (the terminating run has no tiles).  The
// common case, a batch of kBatch slots freed and as many tiles left in the
// current run, takes a straight-line path.
template <class Issue>
QD_HD void stream_refill(StreamLoader& c, int u_limit, const Issue& issue) {
  if (c.issued - c.consumed <= kStreamRing - kBatch && c.u <= u_limit && c.n >= kBatch) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      int slot = c.slot + i;
      if (slot >= kStreamRing) slot -= kStreamRing;
      issue(c.p + (size_t)i * c.stride, slot);
    }
    c.issued += kBatch;
    c.slot += kBatch;
    if (c.slot >= kStreamRing) c.slot -= kStreamRing;
    c.p += (size_t)kBatch * c.stride;
    c.n -= kBatch;
    if (c.n == 0) {
      ++c.run;
      stream_fetch(c);
    }
  }
  while (c.issued - c.consumed < kStreamRing && c.u <= u_limit && c.n > 0) {
    issue(c.p, c.slot);
    ++c.issued;
    c.slot = c.slot + 1 == kStreamRing ? 0 : c.slot + 1;
    c.p += c.stride;
    if (--c.n == 0) {
      ++c.run;
      stream_fetch(c);
    }
  }
}

}  // namespace qd
