// Internal launch interface between the C ABI layer and the HIP kernels.
// Everything here has been validated by the caller (api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace fa {

struct BuildLaunch {
  int kind;
  MaskParams mp;
  int doc_len;
  int Bm, Hm, Q_LEN, KV_LEN, NQB, NKB;
  int block = 128;    // KV_BLOCK_SIZE (a multiple of 128)
  int q_block = 128;  // Q_BLOCK_SIZE (a multiple of 128)
  int* kv_num;
  int* kv_idx;
  int* full_num;
  int* full_idx;
  int* schedule;
  int separate_full;  // 0: every non-empty tile is listed as partial
  // optional per-KV-tile query lists for the backward (all four or none)
  int* q_num;
  int* q_idx;
  int* full_q_num;
  int* full_q_idx;
};

hipError_t launch_build(const BuildLaunch& L, hipStream_t stream);
// validation, schedule and backward lists of caller-given tile lists
hipError_t launch_from_kv_blocks(const BuildLaunch& L, int* status, hipStream_t stream);
int max_build_kv_blocks();

struct FwdLaunch {
  // element strides for b, h, l (d is contiguous)
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  long long sq[3], sk[3], sv[3], so[3];
  int B, Hq, Hkv, Q_LEN, KV_LEN, D;
  int mask_kind;
  MaskParams mp;
  int doc_len;
  int score_kind;
  float softcap;
  const float* slopes;  // device [Hq] or nullptr
  float scale;
  BlockMaskView bm;
  int splits = 1;             // bf16 split-KV slices per item (1: none)
  float* part_o = nullptr;    // workspace [splits][B][Hq][Q_LEN][D] fp32
  float* part_lse = nullptr;  // workspace [splits][B][Hq][Q_LEN] fp32
  // bf16 paged KV (page_table != nullptr): k / v are page caches, sk[0] /
  // sv[0] the page strides; page_table int32 [B][pt_stride]
  const int* page_table = nullptr;
  int page_size = 0, pt_stride = 0, num_pages = 0;
  bool f16 = false;  // 16-bit forward: fp16 inputs (else bf16)
  float* o32 = nullptr;  // 16-bit forward, unsplit: fp32 copy of O [B][Hq][Q_LEN][D]
};

// the 16-bit forward: bf16 or fp16 (L.f16), contiguous or paged K/V (L.page_table)
hipError_t launch_fwd_bf16(const FwdLaunch& L, hipStream_t stream);
// the library's split-KV scratch on the current device (a file-scope device
// array; its address is looked up once per device): no allocation
constexpr size_t kFwdScratchBytes = size_t(32) << 20;
hipError_t fwd_scratch(void** ptr, size_t* bytes);
int fwd_bf16_lds_bytes(int D, int NKB, bool paged);  // LDS of the bf16 forward
constexpr int kMaxLdsBytes = 160 * 1024;
// query rows per workgroup of the fp32 forward (fwd_f32.hip)
constexpr int kF32RowsPerWorkgroup = 8;
constexpr long long kMaxBf16RowStride = 1ll << 22;  // k/v row stride limit of the bf16 forward
hipError_t launch_fwd_f32(const FwdLaunch& L, hipStream_t stream);

struct BwdLaunch {
  // element strides for b, h, l (d is contiguous)
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  float* delta;  // workspace [B][Hq][Q_LEN]
  const float* o32 = nullptr;  // fp32 O [B][Hq][Q_LEN][D]: Delta = dO . O (else recomputed)
  void* dq;
  void* dk;
  void* dv;
  long long sq[3], sk[3], sv[3], sdo[3], sdq[3], sdk[3], sdv[3];
  int B, Hq, Hkv, Q_LEN, KV_LEN, D;
  int mask_kind;
  MaskParams mp;
  int score_kind;
  float softcap;
  const float* slopes;
  float scale;
  BlockMaskView bm;
  const int* q_num;
  const int* q_idx;
  const int* full_q_num;
  const int* full_q_idx;
};

// the 16-bit backward, one object per element type: bf16 or fp16 inputs
hipError_t launch_bwd_bf16(const BwdLaunch& L, hipStream_t stream);
hipError_t launch_bwd_f16(const BwdLaunch& L, hipStream_t stream);

}  // namespace fa
