// CPU replay of the batch-1 streaming step kernel's weight loader
// (qd_stream_plan.h): for every wave of every workgroup the host builds its
// tile runs as the runtime does, the refill and consume calls are made in
// the kernel's order, and each issued tile must be
// the next tile of the wave's expected stream (hence inside its matrix),
// land in the slot the consumer reads it from, be issued before it is
// consumed, never overfill the ring, and the stream must end with every
// issued tile consumed.  Exit status 0 when every case passes.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "qd_stream_plan.h"

using namespace qd;

namespace {

struct Shape {
  const char* name;
  int L, H, Hq, Hkv, D, I, V;
};

struct Tile {
  const unsigned char* p;
  int slot;
};

int g_fail = 0;

void fail(const char* shape, int W, int wg, int wave, const char* what, long idx) {
  if (g_fail < 20)
    std::fprintf(stderr, "FAIL %s W=%d wg=%d wave=%d: %s (tile %ld)\n", shape, W, wg, wave, what,
                 idx);
  ++g_fail;
}

// Bases far apart: pointers are compared, never dereferenced.
const uint16_t* fake_base(int u) {
  return reinterpret_cast<const uint16_t*>((uintptr_t)0x100000000000ull +
                                           (uintptr_t)(u + 1) * 0x10000000000ull);
}

// The wave's tiles in consumption order, from the partition's definition:
// unit by unit, the workgroup's pieces [q*P/W, (q+1)*P/W) of the unit's P
// = R*S pieces, q its index when the W workgroups are listed XCD by XCD
// (workgroup wg runs on XCD wg % 8; q = (wg % 8) * W/8 + wg / 8 when W is a
// multiple of 8, else wg) (piece r: row tile r/S, k-tiles [(r%S)*kps, ...+kps) within
// K), of each the k-tiles kb + wave, kb + wave + 4, ... (the LM head: row
// tile 4g + wave, every k-tile).
std::vector<const unsigned char*> expected(const Shape& sh, int qS, int W, int wg, int wave) {
  std::vector<const unsigned char*> out;
  const int QD = sh.Hq * sh.D, NQKV = (sh.Hq + 2 * sh.Hkv) * sh.D;
  for (int u = 0; u <= 4 * sh.L; ++u) {
    int R, KT, k0, ks, S = 1;
    bool lm = u == 4 * sh.L;
    if (lm) {
      R = sh.V / 64; KT = sh.H / 32; k0 = 0; ks = 1;
    } else {
      const int p = u % 4;
      const int N = p == 0 ? NQKV : p == 1 ? sh.H : p == 2 ? 2 * sh.I : sh.H;
      const int K = p == 0 ? sh.H : p == 1 ? QD : p == 2 ? sh.H : sh.I;
      R = N / 16; KT = K / 32; k0 = wave; ks = 4;
      if (p == 0) S = qS;
    }
    const int kps = (KT + S - 1) / S;
    const long P = (long)R * S;
    long q = wg;
    if (W % 8 == 0) {
      const int per_xcd = W / 8, xcd = wg % 8, slot = wg / 8;
      q = (long)xcd * per_xcd + slot;
    }
    const long r0 = q * P / W, r1 = (q + 1) * P / W;
    const unsigned char* base = reinterpret_cast<const unsigned char*>(fake_base(u));
    const long rows_total = lm ? 4L * R : R;  // row tiles of the matrix
    for (long r = r0; r < r1; ++r) {
      const int kb = (int)(r % S) * kps, ke = kb + kps < KT ? kb + kps : KT;
      for (int k = kb + k0; k < ke; k += ks) {
        const long rt = lm ? 4 * r + wave : r / S;
        if (rt >= rows_total || k >= KT) std::abort();
        out.push_back(base + (rt * KT + k) * 1024);
      }
    }
  }
  return out;
}

void run_wave(const Shape& sh, const StreamArgs& a, int W, int wg, int wave, bool attn_wg) {
  const std::vector<const unsigned char*> want = expected(sh, a.qkv_S, W, wg, wave);
  std::vector<Tile> got;
  std::vector<StreamRun> runs;
  stream_runs(a, W, wg, wave, [&](const unsigned char* p, int n, int stride, int u) {
    if (n > 0xffff || u > 0xffff) fail(sh.name, W, wg, wave, "run fields overflow", n);
    runs.push_back(StreamRun{p, (uint32_t)n | ((uint32_t)u << 16), (uint32_t)stride});
  });
  StreamLoader ld;
  stream_start(ld, runs.data());
  const int u_end = stream_u_end(a);
  auto lim = [&](int u) { return wave == 0 ? u : u_end; };
  auto refill = [&](int u_limit) {
    stream_refill(ld, u_limit, [&](const unsigned char* p, int slot) {
      got.push_back(Tile{p, slot});
    });
    if (ld.issued - ld.consumed > kStreamRing) fail(sh.name, W, wg, wave, "ring overfilled", ld.issued);
    if ((long)got.size() != ld.issued) fail(sh.name, W, wg, wave, "issue count", ld.issued);
  };
  int cs_slot = 0;
  auto consume = [&](int n, int u_limit) {
    refill(u_limit);
    if (ld.issued - ld.consumed < n) fail(sh.name, W, wg, wave, "consumed before issued", ld.consumed);
    for (int i = 0; i < n; ++i) {
      const long j = ld.consumed + i;
      if (j >= (long)got.size() || j >= (long)want.size()) {
        fail(sh.name, W, wg, wave, "past the stream", j);
        return;
      }
      if (got[j].p != want[j]) fail(sh.name, W, wg, wave, "wrong tile", j);
      int slot = cs_slot + i;
      if (slot >= kStreamRing) slot -= kStreamRing;
      if (got[j].slot != slot) fail(sh.name, W, wg, wave, "wrong slot", j);
    }
    ld.consumed += n;
    cs_slot += n;
    if (cs_slot >= kStreamRing) cs_slot -= kStreamRing;
    refill(u_limit);
  };
  // the kernel's projection: per piece (row tile, group), full batches, then singles
  auto project = [&](int u, int u_limit) {
    const StreamShare s = stream_share(a, u, wave, W, wg);
    for (int r = s.r0; r < s.r1; ++r) {
      const int n = stream_piece_tiles(s, r);
      int j = 0;
      for (; j + kBatch <= n; j += kBatch) consume(kBatch, u_limit);
      for (; j < n; ++j) consume(1, u_limit);
    }
  };
  refill(lim(0));
  for (int l = 0; l < a.L; ++l) {
    const int u = 4 * l;
    // a workgroup with attention items loads nothing past QKV until its items ran
    const int lim_qkv = attn_wg ? u + kPrQkv : lim(u + kPrQkv);
    refill(lim_qkv);          // wait for the layer's input
    project(u + kPrQkv, lim_qkv);
    if (!attn_wg) refill(lim(u + kPrO));  // before attention
    refill(lim(u + kPrO));    // wait for attention
    project(u + kPrO, lim(u + kPrO));
    refill(lim(u + kPrGu));
    project(u + kPrGu, lim(u + kPrGu));
    refill(lim(u + kPrDown));
    project(u + kPrDown, lim(u + kPrDown));
  }
  refill(u_end);
  project(u_end - 1, u_end);
  if (ld.issued != ld.consumed) fail(sh.name, W, wg, wave, "tiles left unconsumed", ld.issued);
  if (ld.consumed != (long)want.size()) fail(sh.name, W, wg, wave, "stream length", ld.consumed);
  if (ld.u != u_end || ld.n != 0 || ld.run != &runs.back())
    fail(sh.name, W, wg, wave, "loader not at the end", ld.u);
}

}  // namespace

int main() {
  const Shape shapes[] = {
      {"tiny", 2, 256, 4, 2, 64, 704, 4096},
      {"qwen3-4b", 36, 2560, 32, 8, 128, 9728, 151936},
      {"qwen3-8b", 36, 4096, 32, 8, 128, 12288, 151936},
      {"narrow", 1, 64, 2, 1, 64, 32, 64},      // 2 k-tiles: waves 2, 3 idle
      {"odd", 3, 192, 2, 1, 64, 96, 192},        // rows and k-tiles not multiples of 4
  };
  const int grids[] = {256, 255, 64, 7, 1};
  long cases = 0;
  for (const Shape& sh : shapes) {
    for (int qS : {1, 2, 4}) {
      StreamArgs a{};
      a.L = sh.L; a.H = sh.H; a.QD = sh.Hq * sh.D; a.I = sh.I; a.V = sh.V;
      a.NQKV = (sh.Hq + 2 * sh.Hkv) * sh.D;
      a.qkv_S = qS;
      for (int u = 0; u < 4 * sh.L; ++u) a.w[u] = fake_base(u);
      a.lm = fake_base(4 * sh.L);
      for (int W : grids) {
        if (sh.L > 4 && (W < 64 || qS == 4)) continue;  // large models: realistic cases only
        for (int wg = 0; wg < W; ++wg)
          for (int wave = 0; wave < 4; ++wave)
            for (int attn_wg = 0; attn_wg < 2; ++attn_wg) {
              run_wave(sh, a, W, wg, wave, attn_wg != 0);
              ++cases;
            }
      }
    }
  }
  std::printf("%ld wave streams checked, %d failures\n", cases, g_fail);
  return g_fail == 0 ? 0 : 1;
}
