// Launch plan of the 16-bit forward: how query heads are packed into
// workgroups, which MFMA step the kernel takes, how many work items one launch
// has and how many KV slices fill the chip. The launcher and the C ABI's
// flexattn_fwd_make_plan both call plan_fwd (host code), so the Python
// binding's split count and the kernels' launch shape come from one rule;
// packed_head, the wave -> query head mapping of a packed workgroup, is
// shared by the kernel and a host test.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

constexpr int kPlanWavesPerWorkgroup = 4;  // waves of one forward workgroup

struct FwdPlan {
  int wph = kPlanWavesPerWorkgroup;  // waves per query head: 4 (a 128-row tile), 2 or 1
  int hpw = 1;                       // query heads per workgroup (of one KV group)
  bool r16 = false;                  // 16-row MFMA step (at most 16 query rows per head)
  int packs = 1;                     // workgroups (head packs) per KV group and query tile
  int xcd_round = 0;                 // items per schedule round remapped to XCDs (0: none)
  long long items = 0;               // work items of one unsplit launch
  int splits = 1;                    // suggested KV slices per item
};

// B, Hq, Hkv, Q_LEN, D: the call's shapes. bm_B, bm_H: the BlockMask's batch
// and head extents (1 = broadcast); nqb: its query tile rows, q_block its
// Q_BLOCK_SIZE, nkb its KV tile columns. target: workgroups that fill the
// chip once (two per CU).
inline FwdPlan plan_fwd(int B, int Hq, int Hkv, int Q_LEN, int D, int bm_B, int bm_H, int nqb,
                        int q_block, int nkb, int target) {
  FwdPlan p;
  const int W = kPlanWavesPerWorkgroup;
  const int G = Hq / Hkv;
  // Short query tiles (Q_LEN <= 64, one tile) with the mask broadcast over
  // heads: the fewest waves per head that cover Q_LEN and give a whole
  // number of heads per workgroup inside one KV group.
  if (bm_H == 1 && Q_LEN <= 64)
    for (int w = 1; w < W; w *= 2)
      if (Q_LEN <= 32 * w && G % (W / w) == 0) {
        p.wph = w;
        break;
      }
  // No exact packing (G a multiple of neither 4 nor 2): packs of W / waves
  // heads with a partial last pack per KV group, as long as real heads fill
  // at least half of a group's slots (G = 3, 5, 7, ...). Head dims <= 128
  // only: head dim 256 keeps whole packs (one head per workgroup here).
  if (D <= 128 && bm_H == 1 && Q_LEN <= 64 && p.wph == W) {
    const int w = Q_LEN <= 32 ? 1 : 2;
    if (2 * G > W / w) p.wph = w;
  }
  // At most 16 query rows per head: the 16-row MFMA step (half the matrix
  // work of a 32-row step that would carry 16 empty rows).
  p.r16 = p.wph == 1 && Q_LEN <= 16 && D <= 128;
  p.hpw = W / p.wph;
  p.packs = (G + p.hpw - 1) / p.hpw;
  // XCD-aware order: with the mask broadcast over batch and heads every
  // schedule round holds the B * Hkv * packs items of one query tile; split
  // each round into 8 contiguous chunks of whole KV groups, one per XCD.
  const long long R = (long long)B * Hkv * p.packs;
  p.xcd_round = (bm_B == 1 && bm_H == 1 && R % 8 == 0 && (R / 8) % p.packs == 0 &&
                 R <= 0x7fffffffLL) ? (int)R : 0;
  p.items = R * nqb * (q_block / 128);
  // split-KV: enough slices to fill the chip once when items are few, at
  // most one per listed KV tile and 64; no split when the items already fill
  // half of it
  if (p.items > 0 && p.items < target / 2) {
    long long s = target / p.items;
    if (s > nkb) s = nkb;
    if (s > 64) s = 64;
    p.splits = s < 1 ? 1 : (int)s;
  }
  return p;
}

// Query head of one wave in a packed workgroup. A work item's head index
// counts head packs: packs per KV group = ceil(G / hpw). Wave slot `slot`
// (0 .. hpw - 1) of pack p of KV group hk takes local head p * hpw + slot;
// when G is not a multiple of hpw the group's last pack is partial and its
// spare slots take the group's last head with valid = false (they load and
// synchronise like the others and store nothing). Where hpw divides G this
// is h = item_h * hpw + slot.
struct PackedHead {
  int hk, h;
  bool valid;
};

__host__ __device__ inline PackedHead packed_head(int item_h, int G, int hpw, int slot) {
  const int packs = (G + hpw - 1) / hpw;
  PackedHead r;
  r.hk = item_h / packs;
  const int local = (item_h - r.hk * packs) * hpw + slot;
  r.valid = local < G;
  r.h = r.hk * G + (local < G ? local : G - 1);
  return r;
}

}  // namespace fa
