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
enum StreamProj : int { kPrQkv = 0, kPrO = 1, kPrGu = 2, kPrDown = 3 };

QD_HD int stream_u_end(const StreamArgs& a) { return a.L * kUnitsPerLayer + 1; }

// One wave's share of one unit: the workgroup's row tiles (the LM head:
// 64-row groups) [r0, r1), and of each the k-tiles kstart, kstart + kstep,
// ... (the LM head: row tile 4*g + wave of group g, every k-tile).
struct StreamShare {
  const uint16_t* w;
  int KT, R, r0, r1, kstart, kstep;
  bool lm;
};

// Workgroup wg of W owns rows [wg*R/W, (wg+1)*R/W) of a unit with R row
// tiles (groups).
QD_HD StreamShare stream_share(const StreamArgs& a, int u, int wave, int W, int wg) {
  StreamShare s;
  if (u >= a.L * kUnitsPerLayer) {
    s.w = a.lm; s.KT = a.H / kTileCols; s.R = a.V / kRowsPerGroup;
    s.kstart = 0; s.kstep = 1; s.lm = true;
  } else {
    const int p = u % kUnitsPerLayer;
    s.w = a.w[u];
    s.KT = (p == kPrO ? a.QD : p == kPrDown ? a.I : a.H) / kTileCols;
    s.R = (p == kPrQkv ? a.NQKV : p == kPrGu ? 2 * a.I : a.H) / kTileRows;
    s.kstart = wave; s.kstep = 4; s.lm = false;
  }
  s.r0 = (int)((unsigned)wg * (unsigned)s.R / (unsigned)W);
  s.r1 = (int)((unsigned)(wg + 1) * (unsigned)s.R / (unsigned)W);
  return s;
}

// k-tiles of one row tile (group) that the wave takes.
QD_HD int stream_row_tiles(const StreamShare& s) {
  return s.kstart < s.KT ? (s.KT - s.kstart + s.kstep - 1) / s.kstep : 0;
}

QD_HD const unsigned char* stream_tile(const StreamShare& s, int r, int k, int wave) {
  const int rt = s.lm ? 4 * r + wave : r;
  return reinterpret_cast<const unsigned char*>(s.w) + ((size_t)rt * s.KT + k) * 1024;
}

// The loader's position in the wave's tile stream and the ring counts:
// tiles issued and consumed so far, the slot the next load goes to.
struct StreamLoader {
  int u, r, k;               // unit (u_end: the stream has ended), row tile or group, k-tile
  const unsigned char* p;    // tile (r, k) of this wave; null once the stream has ended
  StreamShare s;
  int issued, consumed, slot;
};

// The first tile of unit u or, when the wave has no share in it, of the
// next unit where it has one.
QD_HD void stream_seek(const StreamArgs& a, StreamLoader& c, int u, int wave, int W, int wg) {
  const int u_end = stream_u_end(a);
  for (; u < u_end; ++u) {
    c.s = stream_share(a, u, wave, W, wg);
    if (c.s.r0 < c.s.r1 && c.s.kstart < c.s.KT) break;
  }
  c.u = u;
  c.r = c.s.r0;
  c.k = c.s.kstart;
  c.p = u < u_end ? stream_tile(c.s, c.r, c.k, wave) : nullptr;
  if (u >= u_end) c.k = c.s.KT;  // no k-tile left: nothing matches a batch
}

QD_HD void stream_advance(const StreamArgs& a, StreamLoader& c, int wave, int W, int wg) {
  c.k += c.s.kstep;
  c.p += (size_t)c.s.kstep * 1024;
  if (c.k < c.s.KT) return;
  c.k = c.s.kstart;
  if (++c.r < c.s.r1) {
    c.p = stream_tile(c.s, c.r, c.k, wave);
    return;
  }
  stream_seek(a, c, c.u + 1, wave, W, wg);
}

QD_HD void stream_start(const StreamArgs& a, StreamLoader& c, int wave, int W, int wg) {
  c.issued = c.consumed = c.slot = 0;
  stream_seek(a, c, 0, wave, W, wg);
}

// Issue loads (issue(tile, slot)) until kStreamRing tiles are loaded or in
// flight ahead of the consumer, but none of a unit after u_limit and none
// past the end of the stream.  The common case, a batch of kBatch slots
// freed and as many tiles left in the current row, takes a straight-line
// path.
template <class Issue>
QD_HD void stream_refill(const StreamArgs& a, StreamLoader& c, int wave, int W, int wg,
                         int u_limit, const Issue& issue) {
  const int u_end = stream_u_end(a);
  if (c.issued - c.consumed <= kStreamRing - kBatch && c.u <= u_limit && c.u < u_end &&
      c.k + (kBatch - 1) * c.s.kstep < c.s.KT) {
    const size_t step = (size_t)c.s.kstep * 1024;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      int slot = c.slot + i;
      if (slot >= kStreamRing) slot -= kStreamRing;
      issue(c.p + i * step, slot);
    }
    c.issued += kBatch;
    c.slot += kBatch;
    if (c.slot >= kStreamRing) c.slot -= kStreamRing;
    c.k += (kBatch - 1) * c.s.kstep;
    c.p += (kBatch - 1) * step;
    stream_advance(a, c, wave, W, wg);
  }
  while (c.issued - c.consumed < kStreamRing && c.u <= u_limit && c.u < u_end) {
    issue(c.p, c.slot);
    ++c.issued;
    c.slot = c.slot + 1 == kStreamRing ? 0 : c.slot + 1;
    stream_advance(a, c, wave, W, wg);
  }
}

}  // namespace qd
