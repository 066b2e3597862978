// kv_shape_check.cpp -- host check of the key-major launch shape (sfag_launch.h): over many
// (live items, head groups) the workgroups of every XCD cover each (head group, live item,
// slice) position exactly once per part, the parts of a split position cover its rows exactly
// once, every extra slot lies inside the workspace's extra area and is written by exactly one
// part, and the reduce's inverse (kv_xslot) names the same slots.  Exit status 0 when all hold.
#include <cstdio>
#include <vector>

#include "sfag_launch.h"

using namespace sfag;

int main() {
  int bad = 0, checked = 0;
  for (int hgc = 1; hgc <= 2; ++hgc)
    for (int citems = 1; citems <= 700; citems += (citems < 80 ? 1 : 7)) {
      const KvShape s = kv_shape(citems, hgc);
      if (s.parts < 1 || s.parts > kKvMaxParts || s.j0 % kKvSlotsPerXcd || s.j0 + s.rem != s.n) ++bad;
      // (hg, citem, slice) -> parts seen; extra slot -> writers
      std::vector<int> seen((size_t)hgc * citems * 8, 0), parts_of((size_t)hgc * citems * 8, 0);
      std::vector<int> xw((size_t)s.extra_slots() + 1, 0);
      for (int xcd = 0; xcd < 8; ++xcd)
        for (int j = 0; j < s.wgs_per_xcd(); ++j) {
          const KvWork w = kv_work(s, xcd, j);
          if (w.citem >= citems) continue;                 // past the live items: exits at once
          if (w.hg < 0 || w.hg >= hgc || w.sl < 0 || w.sl > 7 || w.citem / s.per_xcd != xcd) {
            ++bad;
            continue;
          }
          const size_t key = ((size_t)w.hg * citems + w.citem) * 8 + w.sl;
          seen[key] |= 1 << w.part;
          parts_of[key] = w.nparts;
          const int xs = kv_xslot(s, w.hg, w.citem, w.sl);
          if ((w.nparts > 1) != (xs >= 0) || (w.nparts > 1 && xs != w.xslot)) ++bad;
          if (w.part > 0) {
            const int slot = w.xslot + w.part - 1;
            if (slot < 0 || slot >= s.extra_slots()) ++bad;
            else ++xw[slot];
          }
        }
      for (size_t k = 0; k < seen.size(); ++k)
        if (parts_of[k] < 1 || seen[k] != (1 << parts_of[k]) - 1) ++bad;
      for (int i = 0; i < s.extra_slots(); ++i)
        if (xw[i] > 1) ++bad;
      // row ranges of the parts: consecutive, covering 0 .. nrows - 1 once
      for (int nrows = 0; nrows <= 9; ++nrows) {
        int next = 0;
        for (int p = 0; p < s.parts; ++p) {
          const int r0 = (int)((long long)nrows * p / s.parts), r1 = (int)((long long)nrows * (p + 1) / s.parts);
          if (r0 != next || r1 < r0) ++bad;
          next = r1;
        }
        if (next != nrows) ++bad;
      }
      ++checked;
    }
  std::printf("%s: %d shapes, %d violations\n", bad ? "FAILED" : "ok", checked, bad);
  return bad ? 1 : 0;
}
