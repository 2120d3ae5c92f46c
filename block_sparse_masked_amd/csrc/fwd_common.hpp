// Work-item decoding shared by the forward kernels.
#pragma once

#include "common.hpp"

namespace fa {

struct Item {
  int b, h, qb, mrow;
};

// Map a launch index to (b, h, q-tile) through the BlockMask's schedule.
// The BlockMask may broadcast over batch (Bm == 1) and/or heads (Hm == 1);
// each of its rows then stands for `rep` attention rows, which are visited
// consecutively.
__device__ __forceinline__ Item decode_item(int x, const BlockMaskView& bm, int B, int Hq) {
  const int rep = (B / bm.Bm) * (Hq / bm.Hm);
  const int mrow = bm.schedule[x / rep];
  const int sub = x - (x / rep) * rep;
  const int qb = mrow % bm.NQB;
  const int bh = mrow / bm.NQB;
  const int hm = bh % bm.Hm;
  const int bmi = bh / bm.Hm;
  Item it;
  it.qb = qb;
  it.mrow = mrow;
  if (bm.Bm == 1 && bm.Hm == 1) {
    it.b = sub / Hq;
    it.h = sub - it.b * Hq;
  } else if (bm.Hm == 1) {
    it.b = bmi;
    it.h = sub;
  } else if (bm.Bm == 1) {
    it.b = sub;
    it.h = hm;
  } else {
    it.b = bmi;
    it.h = hm;
  }
  return it;
}

__device__ __forceinline__ float alibi_slope(const float* slopes, int h, int Hq) {
  if (slopes) return slopes[h];
  return exp2f(-8.0f * (float)(h + 1) / (float)Hq);
}

}  // namespace fa
