// Host-side check of the GEMM work assignment (tail split): for many tile
// counts, every (output tile, K step) is computed by exactly one workgroup of
// the launch grid, every tail part writes its own partial slot where the
// fixup kernel looks for it, and tile numbers map one-to-one onto the tiles
// that exist; and the float K-segment index of the concatenated B operand is
// exact for 64-aligned offsets below 2^24.  Exit status 0 on success; the
// first failure is printed.
#include <stdio.h>
#include <stdlib.h>
#include <vector>

#include "gemm.h"

using namespace moe;

struct HostRows {
  std::vector<int> r;
  int rows(int g) const { return r[g]; }
};

static int fail(const char* what, int a, int b) {
  printf("FAIL: %s (%d, %d)\n", what, a, b);
  return 1;
}

static int split_cases = 0;

static int check(const std::vector<int>& rows, int tiles_n, int nk, int P, bool can_split) {
  HostRows a{rows};
  const int groups = (int)rows.size();
  int max_rows = 0;
  for (int r : rows) max_rows = r > max_rows ? r : max_rows;
  const TailPlan p = tail_plan(a, groups, tiles_n, nk, P, can_split);
  int total = 0;
  for (int r : rows) total += (r + 255) / 256 * tiles_n;
  if (p.total != total) return fail("tile count", p.total, total);
  if (p.tail) {
    ++split_cases;
    if (p.tail * p.parts > P || p.tail * p.parts > PART_SLOTS) return fail("parts exceed slots", p.tail, p.parts);
    if (2 * p.tail > P || p.parts < 2 || nk / p.parts < KSPLIT_MIN || nk - nk / p.parts < KSPLIT_GAIN)
      return fail("split rule", p.tail, p.parts);
  }
  const int64_t grid = gemm_grid((int64_t)groups * ((max_rows + 255) / 256) * tiles_n, P);
  std::vector<int> cover((size_t)total * nk, 0), slot_seen(PART_SLOTS, 0);
  for (int64_t bid = 0; bid < grid; ++bid) {
    int t, kb, ke, slot;
    if (!block_work(p, nk, (int)bid, t, kb, ke, slot)) continue;
    if (t < 0 || t >= total) return fail("tile out of range", t, total);
    if (kb < 0 || ke > nk || kb >= ke) return fail("bad K range", kb, ke);
    const int D = total - p.tail;
    if (t < D) {
      if (slot != -1 || kb != 0 || ke != nk) return fail("whole tile split", t, slot);
    } else {
      const int ti = t - D, part = slot - ti * p.parts;
      if (slot < 0 || part < 0 || part >= p.parts) return fail("slot of tail part", t, slot);
      if (kb != part * nk / p.parts || ke != (part + 1) * nk / p.parts) return fail("part K range", kb, ke);
      if (ke - kb < KSPLIT_MIN) return fail("part too short", kb, ke);
      if (slot_seen[slot]++) return fail("slot written twice", slot, t);
    }
    for (int k = kb; k < ke; ++k) cover[(size_t)t * nk + k]++;
  }
  for (size_t i = 0; i < cover.size(); ++i)
    if (cover[i] != 1) return fail("tile/K step covered != once", (int)(i / nk), cover[i]);
  // tile numbers -> existing tiles, one to one
  std::vector<int> seen;
  for (int g = 0; g < groups; ++g) seen.resize(seen.size() + (size_t)((rows[g] + 255) / 256) * tiles_n, 0);
  for (int t = 0; t < total; ++t) {
    int g, tm, tn;
    tile_coords(a, groups, tiles_n, t, g, tm, tn);
    const int mt = (rows[g] + 255) / 256;
    if (g < 0 || g >= groups || tm < 0 || tm >= mt || tn < 0 || tn >= tiles_n) return fail("tile coords", t, g);
    size_t off = 0;
    for (int h = 0; h < g; ++h) off += (size_t)((rows[h] + 255) / 256) * tiles_n;
    if (seen[off + (size_t)tm * tiles_n + tn]++) return fail("tile numbered twice", t, tm);
  }
  return 0;
}

int main() {
  srand(7);
  int cases = 0;
  // the shapes of the layer (experts of a wave, shared / route GEMMs) and random ones
  const int fixed[][5] = {{10946, 10900, 12, 48, 256}, {10946, 10900, 12, 24, 256}, {8192, -1, 14, 96, 256},
                          {8192, -1, 24, 96, 256},     {8192, -1, 24, 72, 256},    {1, 0, 1, 1, 256},
                          {0, 0, 12, 48, 256},         {256, 256, 1, 8, 256},      {300, -1, 3, 64, 8}};
  for (auto& f : fixed) {
    std::vector<int> rows{f[0]};
    if (f[1] >= 0) rows.push_back(f[1]);
    for (int cs = 0; cs < 2; ++cs) {
      if (check(rows, f[2], f[3], f[4], cs)) return 1;
      ++cases;
    }
  }
  for (int i = 0; i < 4000; ++i) {
    const int groups = 1 + rand() % 3;
    std::vector<int> rows(groups);
    for (auto& r : rows) r = rand() % 4 == 0 ? rand() % 300 : rand() % 20000;
    const int tiles_n = 1 + rand() % 30, nk = 1 + rand() % 100;
    const int Ps[] = {256, 255, 240, 64, 8, 3, 1};
    const int P = Ps[rand() % 7];
    if (check(rows, tiles_n, nk, P, rand() % 5 != 0)) return 1;
    ++cases;
  }
  if (split_cases < 100) return fail("too few cases with a tail split", split_cases, cases);
  // The K-segment index of the concatenated B operand, computed in float:
  // exact for every 64-aligned offset below 2^24 and 64-aligned segment length.
  long seg_checks = 0;
  for (int k1 = 64; k1 <= 65536; k1 += (k1 < 4096 ? 64 : 1088)) {
    const float inv = 1.0f / (float)k1;
    const int step = k1 <= 1024 ? 64 : 64 * 7;
    for (int kk = 0; kk < (1 << 24); kk += step) {
      ++seg_checks;
      if (kseg_index(kk, inv) != kk / k1) return fail("K segment index", kk, k1);
    }
    for (int s = 1; (long)s * k1 < (1 << 24); ++s)  // both sides of every boundary
      for (int kk = s * k1 - 64; kk <= s * k1; kk += 64) {
        ++seg_checks;
        if (kseg_index(kk, inv) != kk / k1) return fail("K segment boundary", kk, k1);
      }
  }
  printf("ok %d cases, %d with a tail split, %ld K-segment offsets\n", cases, split_cases, seg_checks);
  return 0;
}
