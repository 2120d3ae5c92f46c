// C ABI of the block-sparse attention library: host-side argument checks,
// then dispatch to the gfx950 kernels on the caller's stream. Every check
// runs before any HIP call, so invalid calls return without touching the
// device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/flexattn.h"
#include "fwd_plan.hpp"
#include "launch.hpp"

static_assert(FLEXATTN_SCRATCH_BYTES == fa::kFwdScratchBytes,
              "the header's scratch size is the library's");

namespace {

thread_local std::string g_last_error;

flexattn_status fail(flexattn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

flexattn_status ok() {
  g_last_error.clear();
  return FLEXATTN_OK;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// BLOCK_SIZE values the builder and the forwards take: multiples of the
// kernels' 128 x 128 tile up to 512 (the backward and from_kv_blocks: 128)
bool valid_block(int block) {
  return block >= fa::kBlock && block <= 4 * fa::kBlock && block % fa::kBlock == 0;
}

// Validate mask kind + params; fill the kernel-side view.
flexattn_status check_mask(flexattn_mask_kind kind, const flexattn_mask_params* p, int B_build,
                           int Q_LEN, int KV_LEN, fa::MaskParams* out, int* doc_len,
                           const char* who) {
  out->window = 0;
  out->sinks = 0;
  out->doc = nullptr;
  out->doc_bstride = 0;
  out->prefix = 0;
  out->nterms = 0;
  for (int t = 0; t < fa::kMaxTerms; ++t) out->terms[t] = 0;
  *doc_len = 0;
  if ((int)kind < FLEXATTN_MASK_NOOP || (int)kind > FLEXATTN_MASK_COMPOSITE)
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: mask_kind %d is not one of the supported kinds", who,
                (int)kind);
  if (kind == FLEXATTN_MASK_SLIDING_SINK) {
    if (!p) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: SLIDING_SINK needs params", who);
    if (p->window < 1)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: SLIDING_SINK window must be >= 1 (got %d)", who,
                  p->window);
    if (p->num_sinks < 0)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: SLIDING_SINK num_sinks must be >= 0 (got %d)",
                  who, p->num_sinks);
    out->window = p->window;
    out->sinks = p->num_sinks;
  }
  if (kind == FLEXATTN_MASK_PREFIX_LM) {
    if (!p) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: PREFIX_LM needs params", who);
    if (p->prefix_len < 0)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: PREFIX_LM prefix_len must be >= 0 (got %d)", who,
                  p->prefix_len);
    out->prefix = p->prefix_len;
  }
  bool needs_doc = kind == FLEXATTN_MASK_DOCUMENT_CAUSAL;
  if (kind == FLEXATTN_MASK_COMPOSITE) {
    if (!p) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: COMPOSITE needs params", who);
    if (p->num_terms < 1 || p->num_terms > fa::kMaxTerms)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: COMPOSITE num_terms must be 1..4 (got %d)", who,
                  p->num_terms);
    int used = 0;
    for (int t = 0; t < p->num_terms; ++t) {
      if (p->terms[t] < 0 || p->terms[t] > 31)
        return fail(FLEXATTN_ERR_INVALID_ARG, "%s: COMPOSITE term %d has bits outside 0..31", who,
                    t);
      used |= p->terms[t];
      out->terms[t] = p->terms[t];
    }
    out->nterms = p->num_terms;
    if ((used & FLEXATTN_PRIM_WINDOW) && p->window < 1)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: COMPOSITE window must be >= 1 (got %d)", who,
                  p->window);
    if ((used & FLEXATTN_PRIM_SINK) && p->num_sinks < 0)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: COMPOSITE num_sinks must be >= 0 (got %d)", who,
                  p->num_sinks);
    if ((used & FLEXATTN_PRIM_PREFIX) && p->prefix_len < 0)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: COMPOSITE prefix_len must be >= 0 (got %d)",
                  who, p->prefix_len);
    out->window = p->window;
    out->sinks = p->num_sinks;
    out->prefix = p->prefix_len;
    needs_doc = (used & FLEXATTN_PRIM_DOCUMENT) != 0;
  }
  if (needs_doc) {
    if (!p) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: DOCUMENT_CAUSAL needs params", who);
    if (!p->doc_ids) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: doc_ids is NULL", who);
    const int need = Q_LEN > KV_LEN ? Q_LEN : KV_LEN;
    if (p->doc_len < need)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: doc_len %d < max(Q_LEN, KV_LEN) = %d", who,
                  p->doc_len, need);
    if (p->doc_batch != 1 && p->doc_batch != B_build)
      return fail(FLEXATTN_ERR_INVALID_ARG,
                  "%s: doc_batch must be 1 or the batch size %d (got %d)", who, B_build,
                  p->doc_batch);
    out->doc = p->doc_ids;
    out->doc_bstride = p->doc_batch > 1 ? (long long)p->doc_len : 0;
    *doc_len = p->doc_len;
  }
  return FLEXATTN_OK;
}

flexattn_status check_tensor(const flexattn_tensor* t, const char* name,
                             const char* who = "flexattn_fwd") {
  if (!t) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: %s is NULL", who, name);
  if (!t->data) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: %s->data is NULL", who, name);
  if (t->dtype != FLEXATTN_F32 && t->dtype != FLEXATTN_BF16 && t->dtype != FLEXATTN_F16)
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: %s dtype %d is not F32, BF16 or F16", who, name,
                (int)t->dtype);
  if (t->B < 1 || t->H < 1 || t->L < 1 || t->D < 1)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: %s has a non-positive extent", who, name);
  if (t->stride[3] != 1)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: %s rows must be contiguous (stride[3]=1)",
                who, name);
  const int es = t->dtype == FLEXATTN_F32 ? 4 : 2;
  if (!aligned16(t->data))
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: %s->data is not 16-byte aligned", who, name);
  for (int i = 0; i < 3; ++i) {
    if (t->stride[i] < 0 || (t->stride[i] * es) % 16 != 0)
      return fail(FLEXATTN_ERR_INVALID_ARG,
                  "%s: %s stride[%d]=%lld is negative or not a multiple of 16 bytes",
                  who, name, i, (long long)t->stride[i]);
  }
  return FLEXATTN_OK;
}

}  // namespace

extern "C" {

const char* flexattn_last_error(void) { return g_last_error.c_str(); }

const char* flexattn_version(void) { return "flexattn-gfx950 0.1.0"; }

flexattn_status flexattn_block_mask_sizes(int32_t B, int32_t H, int32_t Q_LEN, int32_t KV_LEN,
                                          int32_t block, size_t* num_elems, size_t* idx_elems,
                                          size_t* sched_elems) {
  return flexattn_block_mask_sizes_2d(B, H, Q_LEN, KV_LEN, block, block, num_elems, idx_elems,
                                      sched_elems);
}

flexattn_status flexattn_block_mask_sizes_2d(int32_t B, int32_t H, int32_t Q_LEN, int32_t KV_LEN,
                                             int32_t block, int32_t q_block,
                                             size_t* num_elems, size_t* idx_elems,
                                             size_t* sched_elems) {
  if (!num_elems || !idx_elems || !sched_elems)
    return fail(FLEXATTN_ERR_INVALID_ARG, "flexattn_block_mask_sizes: NULL output pointer");
  if (B < 1 || H < 1 || Q_LEN < 1 || KV_LEN < 1)
    return fail(FLEXATTN_ERR_INVALID_ARG,
                "flexattn_block_mask_sizes: B, H, Q_LEN, KV_LEN must be >= 1 (got %d %d %d %d)", B,
                H, Q_LEN, KV_LEN);
  if (!valid_block(block) || !valid_block(q_block))
    return fail(FLEXATTN_ERR_UNSUPPORTED,
                "flexattn_block_mask_sizes: block must be 128, 256, 384 or 512 (got %d, %d)",
                block, q_block);
  const size_t rows = (size_t)B * H * ceil_div(Q_LEN, q_block);
  *num_elems = rows;
  *idx_elems = rows * (size_t)ceil_div(KV_LEN, block);
  *sched_elems = rows;
  return ok();
}

flexattn_status flexattn_create_block_mask(flexattn_mask_kind kind,
                                           const flexattn_mask_params* params, int32_t B,
                                           int32_t H, int32_t Q_LEN, int32_t KV_LEN,
                                           int32_t block, int32_t separate_full_blocks,
                                           flexattn_block_mask* bm, void* stream) {
  static const char* who = "flexattn_create_block_mask";
  if (!bm) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: bm is NULL", who);
  if (B < 1 || H < 1 || Q_LEN < 1 || KV_LEN < 1)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: B, H, Q_LEN, KV_LEN must be >= 1 (got %d %d %d %d)",
                who, B, H, Q_LEN, KV_LEN);
  const int q_block = bm->Q_BLOCK_SIZE > 0 ? bm->Q_BLOCK_SIZE : block;
  if (!valid_block(block) || !valid_block(q_block))
    return fail(FLEXATTN_ERR_UNSUPPORTED,
                "%s: block must be 128, 256, 384 or 512 (got %d, Q_BLOCK_SIZE %d)", who, block,
                q_block);
  const int nkb = ceil_div(KV_LEN, block);
  if (nkb > fa::max_build_kv_blocks())
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: KV_LEN %d exceeds the builder limit of %d tiles",
                who, KV_LEN, fa::max_build_kv_blocks());
  if ((long long)B * H * ceil_div(Q_LEN, q_block) > 0x7fffffffLL / (nkb > 0 ? nkb : 1))
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: index tensor too large", who);
  if (!bm->kv_num_blocks || !bm->kv_indices || !bm->full_kv_num_blocks || !bm->full_kv_indices ||
      !bm->schedule)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: a BlockMask buffer pointer is NULL", who);
  if (bm->q_num_blocks && bm->q_indices && bm->full_q_num_blocks && bm->full_q_indices &&
      (long long)B * H > 0x7fffffffLL)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: B*H=%lld too large for the q_* lists", who,
                (long long)B * H);
  fa::MaskParams mp;
  int doc_len = 0;
  flexattn_status st = check_mask(kind, params, B, Q_LEN, KV_LEN, &mp, &doc_len, who);
  if (st != FLEXATTN_OK) return st;

  bm->B = B;
  bm->H = H;
  bm->Q_LEN = Q_LEN;
  bm->KV_LEN = KV_LEN;
  bm->BLOCK_SIZE = block;
  bm->Q_BLOCK_SIZE = q_block;
  bm->num_q_blocks = ceil_div(Q_LEN, q_block);
  bm->num_kv_blocks = nkb;
  bm->mask_kind = kind;
  if (params) {
    bm->mask_params = *params;
  } else {
    bm->mask_params = flexattn_mask_params{0, 0, nullptr, 0, 0, 0};
  }

  fa::BuildLaunch L;
  L.kind = (int)kind;
  L.mp = mp;
  L.doc_len = doc_len;
  L.Bm = B;
  L.Hm = H;
  L.Q_LEN = Q_LEN;
  L.KV_LEN = KV_LEN;
  L.NQB = bm->num_q_blocks;
  L.NKB = nkb;
  L.kv_num = bm->kv_num_blocks;
  L.kv_idx = bm->kv_indices;
  L.full_num = bm->full_kv_num_blocks;
  L.full_idx = bm->full_kv_indices;
  L.schedule = bm->schedule;
  L.separate_full = separate_full_blocks != 0;
  L.block = block;
  L.q_block = q_block;
  const bool with_q = bm->q_num_blocks && bm->q_indices && bm->full_q_num_blocks &&
                      bm->full_q_indices;
  L.q_num = with_q ? bm->q_num_blocks : nullptr;
  L.q_idx = with_q ? bm->q_indices : nullptr;
  L.full_q_num = with_q ? bm->full_q_num_blocks : nullptr;
  L.full_q_idx = with_q ? bm->full_q_indices : nullptr;
  hipError_t e = fa::launch_build(L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(FLEXATTN_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

flexattn_status flexattn_block_mask_from_kv_blocks(flexattn_block_mask* bm, int32_t* status,
                                                   void* stream) {
  static const char* who = "flexattn_block_mask_from_kv_blocks";
  if (!bm) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: bm is NULL", who);
  if (!status) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: status is NULL", who);
  if (bm->B < 1 || bm->H < 1 || bm->Q_LEN < 1 || bm->KV_LEN < 1)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: B, H, Q_LEN, KV_LEN must be >= 1", who);
  if (bm->BLOCK_SIZE != fa::kBlock || (bm->Q_BLOCK_SIZE != 0 && bm->Q_BLOCK_SIZE != fa::kBlock))
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: BLOCK_SIZE must be 128 (got %d, Q_BLOCK_SIZE %d)",
                who, bm->BLOCK_SIZE, bm->Q_BLOCK_SIZE);
  const int nqb = ceil_div(bm->Q_LEN, fa::kBlock), nkb = ceil_div(bm->KV_LEN, fa::kBlock);
  if (bm->num_q_blocks != nqb || bm->num_kv_blocks != nkb)
    return fail(FLEXATTN_ERR_INVALID_ARG,
                "%s: num_q_blocks / num_kv_blocks must be %d / %d for these lengths", who, nqb,
                nkb);
  if (nkb > fa::max_build_kv_blocks())
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: KV_LEN %d exceeds the builder limit of %d tiles",
                who, bm->KV_LEN, fa::max_build_kv_blocks());
  if ((long long)bm->B * bm->H * nqb > 0x7fffffffLL / (nkb > 0 ? nkb : 1))
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: index tensor too large", who);
  if (!bm->kv_num_blocks || !bm->kv_indices || !bm->full_kv_num_blocks || !bm->full_kv_indices ||
      !bm->schedule)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: a BlockMask buffer pointer is NULL", who);
  fa::MaskParams mp;
  int doc_len = 0;
  flexattn_status st =
      check_mask(bm->mask_kind, &bm->mask_params, bm->B, bm->Q_LEN, bm->KV_LEN, &mp, &doc_len, who);
  if (st != FLEXATTN_OK) return st;
  fa::BuildLaunch L;
  L.kind = (int)bm->mask_kind;
  L.mp = mp;
  L.doc_len = doc_len;
  L.Bm = bm->B;
  L.Hm = bm->H;
  L.Q_LEN = bm->Q_LEN;
  L.KV_LEN = bm->KV_LEN;
  L.NQB = nqb;
  L.NKB = nkb;
  L.kv_num = bm->kv_num_blocks;
  L.kv_idx = bm->kv_indices;
  L.full_num = bm->full_kv_num_blocks;
  L.full_idx = bm->full_kv_indices;
  L.schedule = bm->schedule;
  L.separate_full = 1;
  const bool with_q = bm->q_num_blocks && bm->q_indices && bm->full_q_num_blocks &&
                      bm->full_q_indices;
  L.q_num = with_q ? bm->q_num_blocks : nullptr;
  L.q_idx = with_q ? bm->q_indices : nullptr;
  L.full_q_num = with_q ? bm->full_q_num_blocks : nullptr;
  L.full_q_idx = with_q ? bm->full_q_indices : nullptr;
  hipError_t e = fa::launch_from_kv_blocks(L, status, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(FLEXATTN_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Bytes of split-KV workspace: fp32 O and LSE per slice, query row and head.
size_t splitkv_bytes(long long B, long long Hq, long long Q_LEN, long long D, long long splits) {
  return (size_t)(splits * B * Hq * Q_LEN * (D + 1) * 4);
}

flexattn_status fwd_impl(const flexattn_tensor* q, const flexattn_tensor* k,
                         const flexattn_tensor* v, const flexattn_block_mask* bm,
                         flexattn_score_kind score_kind, const flexattn_score_params* params,
                         float scale, flexattn_tensor* out, float* lse, int splits,
                         void* workspace, size_t workspace_bytes, void* stream, const char* who,
                         const flexattn_page_table* pages = nullptr, float* out_f32 = nullptr) {
  flexattn_status st;
  if ((st = check_tensor(q, "q", who)) != FLEXATTN_OK) return st;
  if ((st = check_tensor(k, "k", who)) != FLEXATTN_OK) return st;
  if ((st = check_tensor(v, "v", who)) != FLEXATTN_OK) return st;
  if ((st = check_tensor(out, "out", who)) != FLEXATTN_OK) return st;
  if (!lse) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: lse is NULL", who);
  if (!bm) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: bm is NULL", who);
  if (k->dtype != q->dtype || v->dtype != q->dtype || out->dtype != q->dtype)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: q, k, v and out must share one dtype", who);
  // head dims: 64 and 128; the 16-bit kernel also 256
  if (q->D != 64 && q->D != 128 && !(q->D == 256 && q->dtype != FLEXATTN_F32))
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: head dim %d is not 64 or 128 (or 256 for 16-bit "
                "inputs)", who, q->D);
  if (k->D != q->D || v->D != q->D || out->D != q->D)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: q, k, v, out head dims differ", who);
  if (out->B != q->B || (!pages && (k->B != q->B || v->B != q->B)))
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: batch sizes differ", who);
  // keys per sequence: the tensors' length, or for a paged cache the
  // BlockMask's KV_LEN (the cache's L is the page size)
  int kv_len = k->L;
  if (pages) {
    if (!pages->page_table || reinterpret_cast<uintptr_t>(pages->page_table) % 4 != 0)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: page_table is NULL or not 4-byte aligned", who);
    if (q->dtype != FLEXATTN_BF16 && q->dtype != FLEXATTN_F16)
      return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: the paged forward is a 16-bit path (bf16 or "
                  "fp16)", who);
    if (k->B != v->B || k->B < 1)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: k and v caches must hold the same pages", who);
    if (k->L % fa::kBlock != 0)
      return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: page size %d is not a multiple of 128", who,
                  k->L);
    if (!bm) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: bm is NULL", who);
    kv_len = bm->KV_LEN;
    if (kv_len < 1 || pages->max_pages < 1 ||
        (long long)pages->max_pages * k->L < (long long)kv_len)
      return fail(FLEXATTN_ERR_INVALID_ARG,
                  "%s: max_pages=%d pages of %d keys do not cover KV_LEN=%d", who,
                  pages->max_pages, k->L, kv_len);
  }
  if (k->H != v->H || out->H != q->H)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: head counts of k/v or q/out differ", who);
  if (q->H % k->H != 0)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: Hq=%d is not a multiple of Hkv=%d", who, q->H,
                k->H);
  if (k->L != v->L) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: k and v lengths differ", who);
  (void)kv_len;
  if (out->L != q->L) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: out and q lengths differ", who);
  if (!(std::isfinite(scale)))
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: scale is not finite", who);
  // BlockMask consistency
  if (!valid_block(bm->BLOCK_SIZE))
    return fail(FLEXATTN_ERR_UNSUPPORTED,
                "%s: BlockMask BLOCK_SIZE must be 128, 256, 384 or 512 (got %d)", who,
                bm->BLOCK_SIZE);
  const int BS = bm->BLOCK_SIZE;
  const int QBS = bm->Q_BLOCK_SIZE > 0 ? bm->Q_BLOCK_SIZE : BS;
  if (!valid_block(QBS))
    return fail(FLEXATTN_ERR_UNSUPPORTED,
                "%s: BlockMask Q_BLOCK_SIZE must be 128, 256, 384 or 512 (got %d)", who, QBS);
  if (bm->Q_LEN != q->L || bm->KV_LEN != kv_len)
    return fail(FLEXATTN_ERR_INVALID_ARG,
                "%s: BlockMask built for Q_LEN=%d KV_LEN=%d, tensors have %d and %d", who,
                bm->Q_LEN, bm->KV_LEN, q->L, kv_len);
  if (bm->num_q_blocks != ceil_div(q->L, QBS) || bm->num_kv_blocks != ceil_div(kv_len, BS))
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: BlockMask tile counts do not match its lengths",
                who);
  if (!(bm->B == 1 || bm->B == q->B) || !(bm->H == 1 || bm->H == q->H))
    return fail(FLEXATTN_ERR_INVALID_ARG,
                "%s: BlockMask extents (B=%d, H=%d) must be 1 or match q (B=%d, H=%d)", who, bm->B,
                bm->H, q->B, q->H);
  if (!bm->kv_num_blocks || !bm->kv_indices || !bm->full_kv_num_blocks || !bm->full_kv_indices ||
      !bm->schedule)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: a BlockMask buffer pointer is NULL", who);
  fa::MaskParams mp;
  int doc_len = 0;
  if ((st = check_mask(bm->mask_kind, &bm->mask_params, q->B, q->L, kv_len, &mp, &doc_len, who)) !=
      FLEXATTN_OK)
    return st;
  if (mp.doc && bm->mask_params.doc_batch > 1 && bm->B != q->B)
    return fail(FLEXATTN_ERR_INVALID_ARG,
                "%s: per-batch doc_ids need a BlockMask built per batch (B=%d)", who, q->B);
  // the fp32 kernel launches BLOCK_SIZE / 32 workgroups per tile row, the
  // 16-bit one BLOCK_SIZE / 128 per tile row and head
  if ((long long)q->B * q->H * bm->num_q_blocks * (QBS / 32) > 0x7fffffffLL)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: too many query tiles for one launch", who);
  if ((int)score_kind < FLEXATTN_SCORE_NONE || (int)score_kind > FLEXATTN_SCORE_SOFTCAP_ALIBI)
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: score_kind %d is not a supported kind", who,
                (int)score_kind);
  float softcap = 0.0f;
  const float* slopes = nullptr;
  if (score_kind == FLEXATTN_SCORE_SOFTCAP || score_kind == FLEXATTN_SCORE_SOFTCAP_ALIBI) {
    if (!params || !(params->softcap > 0.0f) || !std::isfinite(params->softcap))
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: softcap must be a finite value > 0", who);
    softcap = params->softcap;
  }
  if (score_kind == FLEXATTN_SCORE_ALIBI || score_kind == FLEXATTN_SCORE_SOFTCAP_ALIBI)
    slopes = params ? params->alibi_slopes : nullptr;

  const bool half = q->dtype == FLEXATTN_BF16 || q->dtype == FLEXATTN_F16;  // 16-bit kernel
  if (half && fa::fwd_bf16_lds_bytes(q->D, bm->num_kv_blocks * (BS / fa::kBlock), pages != nullptr) >
                                        fa::kMaxLdsBytes)
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: KV_LEN %d needs more LDS than a workgroup has", who,
                kv_len);
  // the bf16 kernel addresses a block of up to 128 key rows with 32-bit offsets
  if (half &&
      (k->stride[2] > fa::kMaxBf16RowStride || v->stride[2] > fa::kMaxBf16RowStride))
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: k/v row stride above %lld elements", who,
                (long long)fa::kMaxBf16RowStride);
  if (splits > 1) {
    if (!half)
      return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: split-KV is a bf16 / fp16 path", who);
    if (splits > 256)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: num_splits %d above 256", who, splits);
    if (!workspace || !aligned16(workspace))
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: workspace is NULL or not 16-byte aligned", who);
    if (workspace_bytes < splitkv_bytes(q->B, q->H, q->L, q->D, splits))
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: workspace of %zu bytes is below the %zu needed",
                  who, workspace_bytes, splitkv_bytes(q->B, q->H, q->L, q->D, splits));
    if ((long long)q->B * q->H * bm->num_q_blocks * (QBS / fa::kBlock) * splits > 0x7fffffffLL)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: too many workgroups for one launch", who);
  }
  fa::FwdLaunch L;
  L.q = q->data;
  L.k = k->data;
  L.v = v->data;
  L.o = out->data;
  L.lse = lse;
  for (int i = 0; i < 3; ++i) {
    L.sq[i] = q->stride[i];
    L.sk[i] = k->stride[i];
    L.sv[i] = v->stride[i];
    L.so[i] = out->stride[i];
  }
  L.B = q->B;
  L.Hq = q->H;
  L.Hkv = k->H;
  L.Q_LEN = q->L;
  L.KV_LEN = kv_len;
  L.D = q->D;
  L.mask_kind = (int)bm->mask_kind;
  L.mp = mp;
  L.doc_len = doc_len;
  L.score_kind = (int)score_kind;
  L.softcap = softcap;
  L.slopes = slopes;
  L.scale = scale;
  L.bm.kv_num = bm->kv_num_blocks;
  L.bm.kv_idx = bm->kv_indices;
  L.bm.full_num = bm->full_kv_num_blocks;
  L.bm.full_idx = bm->full_kv_indices;
  L.bm.schedule = bm->schedule;
  L.bm.Bm = bm->B;
  L.bm.Hm = bm->H;
  L.bm.NQB = bm->num_q_blocks;
  L.bm.NKB = bm->num_kv_blocks;
  L.bm.BS = BS;
  L.bm.QBS = QBS;
  if (out_f32) {
    if (!half || splits > 1 || pages || !aligned16(out_f32))
      return fail(FLEXATTN_ERR_INVALID_ARG,
                  "%s: out_f32 needs a 16-bit, unsplit, contiguous-KV call and 16-byte alignment",
                  who);
    L.o32 = out_f32;
  }
  if (pages) {
    L.page_table = pages->page_table;
    L.page_size = k->L;
    L.pt_stride = pages->max_pages;
    L.num_pages = k->B;
  }
  if (splits > 1) {
    L.splits = splits;
    L.part_o = static_cast<float*>(workspace);
    L.part_lse = L.part_o + (size_t)splits * q->B * q->H * q->L * q->D;
  }
  L.f16 = q->dtype == FLEXATTN_F16;
  hipError_t e = half
                     ? fa::launch_fwd_bf16(L, static_cast<hipStream_t>(stream))
                     : fa::launch_fwd_f32(L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(FLEXATTN_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

flexattn_status flexattn_fwd(const flexattn_tensor* q, const flexattn_tensor* k,
                             const flexattn_tensor* v, const flexattn_block_mask* bm,
                             flexattn_score_kind score_kind, const flexattn_score_params* params,
                             float scale, flexattn_tensor* out, float* lse, void* stream) {
  return fwd_impl(q, k, v, bm, score_kind, params, scale, out, lse, 1, nullptr, 0, stream,
                  "flexattn_fwd");
}

flexattn_status flexattn_fwd_make_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t Q_LEN,
                                       int32_t D, flexattn_dtype dtype,
                                       const flexattn_block_mask* bm, int32_t target_workgroups,
                                       flexattn_fwd_plan* plan) {
  static const char* who = "flexattn_fwd_make_plan";
  if (!bm || !plan) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: bm or plan is NULL", who);
  if (B < 1 || Hq < 1 || Hkv < 1 || Q_LEN < 1 || D < 1)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: non-positive shape", who);
  if (Hq % Hkv != 0)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: Hq=%d is not a multiple of Hkv=%d", who, Hq, Hkv);
  if (dtype != FLEXATTN_F32 && dtype != FLEXATTN_BF16 && dtype != FLEXATTN_F16)
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: dtype %d is not F32, BF16 or F16", who,
                (int)dtype);
  if (!valid_block(bm->BLOCK_SIZE))
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: BlockMask BLOCK_SIZE %d", who, bm->BLOCK_SIZE);
  const int QBS = bm->Q_BLOCK_SIZE > 0 ? bm->Q_BLOCK_SIZE : bm->BLOCK_SIZE;
  if (!valid_block(QBS))
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: BlockMask Q_BLOCK_SIZE %d", who, QBS);
  if (!(bm->B == 1 || bm->B == B) || !(bm->H == 1 || bm->H == Hq) || bm->Q_LEN != Q_LEN ||
      bm->num_q_blocks != ceil_div(Q_LEN, QBS) || bm->num_kv_blocks < 1)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: BlockMask does not match the shapes", who);
  const int target = target_workgroups > 0 ? target_workgroups : 512;
  if (dtype == FLEXATTN_F32) {
    plan->waves_per_head = 0;  // not the 16-bit kernel's layout: 8-row workgroups
    plan->heads_per_workgroup = 1;
    plan->row16 = 0;
    plan->num_splits = 1;
    plan->work_items = (int64_t)B * Hq * bm->num_q_blocks * (QBS / fa::kF32RowsPerWorkgroup);
    return ok();
  }
  const fa::FwdPlan p = fa::plan_fwd(B, Hq, Hkv, Q_LEN, D, bm->B, bm->H, bm->num_q_blocks, QBS,
                                     bm->num_kv_blocks, target);
  plan->waves_per_head = p.wph;
  plan->heads_per_workgroup = p.hpw;
  plan->row16 = p.r16 ? 1 : 0;
  plan->num_splits = p.splits;
  plan->work_items = p.items;
  return ok();
}

size_t flexattn_fwd_splitkv_workspace_bytes(int32_t B, int32_t Hq, int32_t Q_LEN, int32_t D,
                                            int32_t num_splits) {
  if (B < 1 || Hq < 1 || Q_LEN < 1 || D < 1 || num_splits < 1) return 0;
  return splitkv_bytes(B, Hq, Q_LEN, D, num_splits);
}

flexattn_status flexattn_fwd_splitkv(const flexattn_tensor* q, const flexattn_tensor* k,
                                     const flexattn_tensor* v, const flexattn_block_mask* bm,
                                     flexattn_score_kind score_kind,
                                     const flexattn_score_params* params, float scale,
                                     int32_t num_splits, void* workspace, size_t workspace_bytes,
                                     flexattn_tensor* out, float* lse, void* stream) {
  static const char* who = "flexattn_fwd_splitkv";
  if (num_splits < 1)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: num_splits must be >= 1 (got %d)", who,
                num_splits);
  return fwd_impl(q, k, v, bm, score_kind, params, scale, out, lse, num_splits, workspace,
                  workspace_bytes, stream, who);
}

flexattn_status flexattn_fwd_splitkv_noalloc(const flexattn_tensor* q, const flexattn_tensor* k,
                                             const flexattn_tensor* v,
                                             const flexattn_block_mask* bm,
                                             flexattn_score_kind score_kind,
                                             const flexattn_score_params* params, float scale,
                                             int32_t num_splits, flexattn_tensor* out, float* lse,
                                             void* stream) {
  static const char* who = "flexattn_fwd_splitkv_noalloc";
  if (num_splits < 1)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: num_splits must be >= 1 (got %d)", who,
                num_splits);
  if (!q) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: q is NULL", who);
  const size_t need = num_splits > 1 ? splitkv_bytes(q->B, q->H, q->L, q->D, num_splits) : 0;
  if (need > fa::kFwdScratchBytes)
    return fail(FLEXATTN_ERR_INVALID_ARG,
                "%s: %d slices of B=%d Hq=%d Q_LEN=%d D=%d need %zu bytes of scratch; the "
                "library's scratch holds %zu (use flexattn_fwd_splitkv with a workspace, or "
                "fewer slices)", who, num_splits, q->B, q->H, q->L, q->D, need,
                fa::kFwdScratchBytes);
  if (stream) {
    int dev = 0, sdev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return fail(FLEXATTN_ERR_HIP, "%s: cannot query the stream's device", who);
    if (dev != sdev)
      return fail(FLEXATTN_ERR_INVALID_ARG,
                  "%s: the stream belongs to device %d, the current device is %d", who, sdev,
                  dev);
  }
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (num_splits > 1) {
    const hipError_t e = fa::fwd_scratch(&ws, &ws_bytes);
    if (e != hipSuccess)
      return fail(FLEXATTN_ERR_HIP, "%s: scratch lookup failed: %s", who, hipGetErrorString(e));
  }
  return fwd_impl(q, k, v, bm, score_kind, params, scale, out, lse, num_splits, ws, ws_bytes,
                  stream, who);
}

flexattn_status flexattn_fwd_train(const flexattn_tensor* q, const flexattn_tensor* k,
                                   const flexattn_tensor* v, const flexattn_block_mask* bm,
                                   flexattn_score_kind score_kind,
                                   const flexattn_score_params* params, float scale,
                                   flexattn_tensor* out, float* lse, float* out_f32,
                                   void* stream) {
  static const char* who = "flexattn_fwd_train";
  if (!out_f32) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: out_f32 is NULL", who);
  return fwd_impl(q, k, v, bm, score_kind, params, scale, out, lse, 1, nullptr, 0, stream, who,
                  nullptr, out_f32);
}

flexattn_status flexattn_fwd_paged(const flexattn_tensor* q, const flexattn_tensor* k_cache,
                                   const flexattn_tensor* v_cache,
                                   const flexattn_page_table* pages,
                                   const flexattn_block_mask* bm, flexattn_score_kind score_kind,
                                   const flexattn_score_params* params, float scale,
                                   int32_t num_splits, void* workspace, size_t workspace_bytes,
                                   flexattn_tensor* out, float* lse, void* stream) {
  static const char* who = "flexattn_fwd_paged";
  if (!pages) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: pages is NULL", who);
  if (num_splits < 1)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: num_splits must be >= 1 (got %d)", who,
                num_splits);
  return fwd_impl(q, k_cache, v_cache, bm, score_kind, params, scale, out, lse, num_splits,
                  workspace, workspace_bytes, stream, who, pages);
}

static flexattn_status bwd_impl(const flexattn_tensor* q, const flexattn_tensor* k,
                                const flexattn_tensor* v, const float* lse, const float* out_f32,
                                const flexattn_tensor* d_out, const flexattn_block_mask* bm,
                                flexattn_score_kind score_kind,
                                const flexattn_score_params* params, float scale,
                                flexattn_tensor* dq, flexattn_tensor* dk, flexattn_tensor* dv,
                                float* workspace, void* stream, const char* who) {
  flexattn_status st;
  const flexattn_tensor* all[7] = {q, k, v, d_out, dq, dk, dv};
  const char* names[7] = {"q", "k", "v", "d_out", "dq", "dk", "dv"};
  for (int i = 0; i < 7; ++i)
    if ((st = check_tensor(all[i], names[i], who)) != FLEXATTN_OK) return st;
  if (q->dtype != FLEXATTN_BF16 && q->dtype != FLEXATTN_F16)
    return fail(FLEXATTN_ERR_UNSUPPORTED,
                "%s: q must be BF16 or F16 (the backward is a 16-bit path)", who);
  for (int i = 1; i < 7; ++i)
    if (all[i]->dtype != q->dtype)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: %s dtype differs from q", who, names[i]);
  if (!lse) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: lse is NULL", who);
  if (!workspace) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: workspace is NULL", who);
  if (!bm) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: bm is NULL", who);
  if (q->D != 64 && q->D != 128)
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: head dim %d is not 64 or 128", who, q->D);
  for (int i = 1; i < 7; ++i)
    if (all[i]->D != q->D || all[i]->B != q->B)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: %s batch or head dim differs from q", who,
                  names[i]);
  const flexattn_tensor* qlike[2] = {d_out, dq};
  for (int i = 0; i < 2; ++i)
    if (qlike[i]->H != q->H || qlike[i]->L != q->L)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: d_out and dq must be shaped like q", who);
  const flexattn_tensor* kvlike[3] = {v, dk, dv};
  for (int i = 0; i < 3; ++i)
    if (kvlike[i]->H != k->H || kvlike[i]->L != k->L)
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: v, dk and dv must be shaped like k", who);
  if (q->H % k->H != 0)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: Hq=%d is not a multiple of Hkv=%d", who, q->H,
                k->H);
  if (!std::isfinite(scale)) return fail(FLEXATTN_ERR_INVALID_ARG, "%s: scale is not finite", who);
  if (!valid_block(bm->BLOCK_SIZE))
    return fail(FLEXATTN_ERR_UNSUPPORTED,
                "%s: BlockMask BLOCK_SIZE must be 128, 256, 384 or 512 (got %d)", who,
                bm->BLOCK_SIZE);
  const int BS = bm->BLOCK_SIZE;
  const int QBS = bm->Q_BLOCK_SIZE > 0 ? bm->Q_BLOCK_SIZE : BS;
  if (!valid_block(QBS))
    return fail(FLEXATTN_ERR_UNSUPPORTED,
                "%s: BlockMask Q_BLOCK_SIZE must be 128, 256, 384 or 512 (got %d)", who, QBS);
  if (bm->Q_LEN != q->L || bm->KV_LEN != k->L || bm->num_q_blocks != ceil_div(q->L, QBS) ||
      bm->num_kv_blocks != ceil_div(k->L, BS))
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: BlockMask lengths do not match the tensors", who);
  if (!(bm->B == 1 || bm->B == q->B) || !(bm->H == 1 || bm->H == q->H))
    return fail(FLEXATTN_ERR_INVALID_ARG,
                "%s: BlockMask extents (B=%d, H=%d) must be 1 or match q (B=%d, H=%d)", who, bm->B,
                bm->H, q->B, q->H);
  if (!bm->kv_num_blocks || !bm->kv_indices || !bm->full_kv_num_blocks || !bm->full_kv_indices ||
      !bm->schedule)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: a BlockMask buffer pointer is NULL", who);
  if (!bm->q_num_blocks || !bm->q_indices || !bm->full_q_num_blocks || !bm->full_q_indices)
    return fail(FLEXATTN_ERR_INVALID_ARG,
                "%s: the BlockMask has no q_* lists (build it with the q_* buffers set)", who);
  fa::MaskParams mp;
  int doc_len = 0;
  if ((st = check_mask(bm->mask_kind, &bm->mask_params, q->B, q->L, k->L, &mp, &doc_len, who)) !=
      FLEXATTN_OK)
    return st;
  if (mp.doc && bm->mask_params.doc_batch > 1 && bm->B != q->B)
    return fail(FLEXATTN_ERR_INVALID_ARG,
                "%s: per-batch doc_ids need a BlockMask built per batch (B=%d)", who, q->B);
  if ((long long)q->B * q->H * bm->num_q_blocks * (QBS / fa::kBlock) > 0x7fffffffLL ||
      (long long)q->B * k->H * bm->num_kv_blocks * (BS / fa::kBlock) > 0x7fffffffLL ||
      (long long)q->B * q->H * q->L > 0x7fffffffLL)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: too many tiles or rows for one launch", who);
  if ((int)score_kind < FLEXATTN_SCORE_NONE || (int)score_kind > FLEXATTN_SCORE_SOFTCAP_ALIBI)
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: score_kind %d is not a supported kind", who,
                (int)score_kind);
  float softcap = 0.0f;
  const float* slopes = nullptr;
  if (score_kind == FLEXATTN_SCORE_SOFTCAP || score_kind == FLEXATTN_SCORE_SOFTCAP_ALIBI) {
    if (!params || !(params->softcap > 0.0f) || !std::isfinite(params->softcap))
      return fail(FLEXATTN_ERR_INVALID_ARG, "%s: softcap must be a finite value > 0", who);
    softcap = params->softcap;
  }
  if (score_kind == FLEXATTN_SCORE_ALIBI || score_kind == FLEXATTN_SCORE_SOFTCAP_ALIBI)
    slopes = params ? params->alibi_slopes : nullptr;
  // the backward kernels address a tile of up to 128 rows of q, k, v and
  // d_out with 32-bit offsets
  if (q->stride[2] > fa::kMaxBf16RowStride || d_out->stride[2] > fa::kMaxBf16RowStride ||
      k->stride[2] > fa::kMaxBf16RowStride || v->stride[2] > fa::kMaxBf16RowStride)
    return fail(FLEXATTN_ERR_UNSUPPORTED, "%s: q/k/v/d_out row stride above %lld elements", who,
                (long long)fa::kMaxBf16RowStride);

  fa::BwdLaunch L;
  L.q = q->data;
  L.k = k->data;
  L.v = v->data;
  L.dout = d_out->data;
  L.lse = lse;
  L.delta = workspace;
  L.o32 = out_f32;
  L.dq = dq->data;
  L.dk = dk->data;
  L.dv = dv->data;
  for (int i = 0; i < 3; ++i) {
    L.sq[i] = q->stride[i];
    L.sk[i] = k->stride[i];
    L.sv[i] = v->stride[i];
    L.sdo[i] = d_out->stride[i];
    L.sdq[i] = dq->stride[i];
    L.sdk[i] = dk->stride[i];
    L.sdv[i] = dv->stride[i];
  }
  L.B = q->B;
  L.Hq = q->H;
  L.Hkv = k->H;
  L.Q_LEN = q->L;
  L.KV_LEN = k->L;
  L.D = q->D;
  L.mask_kind = (int)bm->mask_kind;
  L.mp = mp;
  L.score_kind = (int)score_kind;
  L.softcap = softcap;
  L.slopes = slopes;
  L.scale = scale;
  L.bm.kv_num = bm->kv_num_blocks;
  L.bm.kv_idx = bm->kv_indices;
  L.bm.full_num = bm->full_kv_num_blocks;
  L.bm.full_idx = bm->full_kv_indices;
  L.bm.schedule = bm->schedule;
  L.bm.Bm = bm->B;
  L.bm.Hm = bm->H;
  L.bm.NQB = bm->num_q_blocks;
  L.bm.NKB = bm->num_kv_blocks;
  L.bm.BS = BS;
  L.bm.QBS = QBS;
  L.q_num = bm->q_num_blocks;
  L.q_idx = bm->q_indices;
  L.full_q_num = bm->full_q_num_blocks;
  L.full_q_idx = bm->full_q_indices;
  hipError_t e = q->dtype == FLEXATTN_F16
                     ? fa::launch_bwd_f16(L, static_cast<hipStream_t>(stream))
                     : fa::launch_bwd_bf16(L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(FLEXATTN_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ok();
}

flexattn_status flexattn_bwd(const flexattn_tensor* q, const flexattn_tensor* k,
                             const flexattn_tensor* v, const float* lse,
                             const flexattn_tensor* d_out,
                             const flexattn_block_mask* bm, flexattn_score_kind score_kind,
                             const flexattn_score_params* params, float scale,
                             flexattn_tensor* dq, flexattn_tensor* dk, flexattn_tensor* dv,
                             float* workspace, void* stream) {
  return bwd_impl(q, k, v, lse, nullptr, d_out, bm, score_kind, params, scale, dq, dk, dv,
                  workspace, stream, "flexattn_bwd");
}

flexattn_status flexattn_bwd_from_out(const flexattn_tensor* q, const flexattn_tensor* k,
                                      const flexattn_tensor* v, const float* lse,
                                      const float* out_f32, const flexattn_tensor* d_out,
                                      const flexattn_block_mask* bm,
                                      flexattn_score_kind score_kind,
                                      const flexattn_score_params* params, float scale,
                                      flexattn_tensor* dq, flexattn_tensor* dk,
                                      flexattn_tensor* dv, float* workspace, void* stream) {
  static const char* who = "flexattn_bwd_from_out";
  if (!out_f32 || reinterpret_cast<uintptr_t>(out_f32) % 16 != 0)
    return fail(FLEXATTN_ERR_INVALID_ARG, "%s: out_f32 is NULL or not 16-byte aligned", who);
  return bwd_impl(q, k, v, lse, out_f32, d_out, bm, score_kind, params, scale, dq, dk, dv,
                  workspace, stream, who);
}

}  // extern "C"
