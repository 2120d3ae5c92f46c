// Exhaustive host check of the forward's head packing (fa::packed_head, the
// function the kernel calls): for group sizes 1..8 and packs of 1, 2 and 4
// heads, every query head of every KV group is taken by exactly one valid
// wave slot, that slot's KV head is h / G, and every spare slot is invalid
// and names a head of its own group. Prints "ok" or the first mismatch.
#include <cstdio>
#include <vector>

#include "fwd_plan.hpp"

int main() {
  const int Hkv = 3;
  for (int G = 1; G <= 8; ++G)
    for (int hpw : {1, 2, 4}) {
      const int packs = (G + hpw - 1) / hpw;
      std::vector<int> seen(Hkv * G, 0);
      for (int item_h = 0; item_h < Hkv * packs; ++item_h)
        for (int slot = 0; slot < hpw; ++slot) {
          const fa::PackedHead p = fa::packed_head(item_h, G, hpw, slot);
          if (p.hk != item_h / packs || p.h / G != p.hk || p.h < 0 || p.h >= Hkv * G) {
            std::printf("bad head: G=%d hpw=%d item=%d slot=%d -> hk=%d h=%d\n", G, hpw, item_h,
                        slot, p.hk, p.h);
            return 1;
          }
          if (p.valid) ++seen[p.h];
          if (G % hpw == 0 && (!p.valid || p.h != item_h * hpw + slot)) {
            std::printf("whole packs differ: G=%d hpw=%d item=%d slot=%d\n", G, hpw, item_h, slot);
            return 1;
          }
        }
      for (int h = 0; h < Hkv * G; ++h)
        if (seen[h] != 1) {
          std::printf("head %d stored %d times (G=%d hpw=%d)\n", h, seen[h], G, hpw);
          return 1;
        }
    }
  std::printf("ok\n");
  return 0;
}
