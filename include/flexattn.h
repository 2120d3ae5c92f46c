/*
 * flexattn.h - C ABI of the MI355X (gfx950) FlexAttention-style block-sparse
 * attention forward: a BlockMask builder and a tiled block-sparse forward.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named "device" are HIP device pointers; everything else is host.
 * - The caller owns and allocates every buffer (inputs, outputs and the
 *   BlockMask index tensors, sized with flexattn_block_mask_sizes). The
 *   library allocates no device memory, keeps no state between calls and
 *   never frees caller memory.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   All device work is enqueued on it asynchronously: no host
 *   synchronisation and no device-to-host copy, so the calls can be captured
 *   in a HIP graph.
 * - Every argument is checked on the host before any HIP call. A bad
 *   argument returns FLEXATTN_ERR_INVALID_ARG (bad pointer, shape, stride,
 *   alignment) or FLEXATTN_ERR_UNSUPPORTED (a dtype, head dim, block size or
 *   kind outside the supported set) and sets a thread-local message read by
 *   flexattn_last_error(); nothing is launched. A failed launch returns
 *   FLEXATTN_ERR_HIP. No C++ exception crosses this boundary.
 * - Index tensors are int32; layouts are row-major (C order).
 */
#ifndef FLEXATTN_H
#define FLEXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Status of every entry point. The values are small positive integers (0 =
 * success) so that a C caller can test `if (status)`; they are part of the
 * ABI and do not change.
 *   FLEXATTN_OK               the call was checked and its work enqueued.
 *   FLEXATTN_ERR_INVALID_ARG  a pointer, shape, stride or alignment is wrong;
 *                             nothing was launched.
 *   FLEXATTN_ERR_UNSUPPORTED  a valid request outside the built set (dtype,
 *                             head dim, block size, kind, size limit);
 *                             nothing was launched.
 *   FLEXATTN_ERR_HIP          a HIP call or kernel launch failed.
 */
typedef enum {
  FLEXATTN_OK = 0,
  FLEXATTN_ERR_INVALID_ARG = 1,
  FLEXATTN_ERR_UNSUPPORTED = 2,
  FLEXATTN_ERR_HIP = 3
} flexattn_status;

/*
 * mask_mod kinds: a fixed, enumerated set of element masks
 * allowed(b, h, q_idx, kv_idx) -> bool, true = the pair may attend
 * (page "tensorplay.nn.attention API", section create_block_mask, the
 * mask_mod parameter and the causal_mask example; noop_mask; and_masks and
 * or_masks compose the sliding-window kind).
 *   NOOP             every pair.
 *   CAUSAL           kv_idx <= q_idx.
 *   SLIDING_SINK     kv_idx <= q_idx AND (q_idx - kv_idx < window OR
 *                    kv_idx < num_sinks): a sliding window plus StreamingLLM
 *                    sink tokens (page "transformerlab", section "Attention
 *                    variants", rows local_flex and sink).
 *   DOCUMENT_CAUSAL  doc[q_idx] == doc[kv_idx] AND kv_idx <= q_idx: causal
 *                    attention inside each packed document, the
 *                    block-diagonal mask of page "Attention Backends"
 *                    (section "Why care about Attention Kernels?").
 *   PREFIX_LM        kv_idx < prefix_len OR kv_idx <= q_idx: every query sees
 *                    the whole prefix, causal after it (PrefixLM, named on
 *                    the same page and section).
 *   COMPOSITE        runtime composition (page "tensorplay.nn.attention API":
 *                    or_masks is the union, and_masks the intersection of
 *                    mask_mods): the OR of num_terms (1..4) terms, each the
 *                    AND of the primitives its bit set selects:
 *                      FLEXATTN_PRIM_CAUSAL    kv_idx <= q_idx
 *                      FLEXATTN_PRIM_WINDOW    q_idx - kv_idx < window
 *                      FLEXATTN_PRIM_SINK      kv_idx < num_sinks
 *                      FLEXATTN_PRIM_PREFIX    kv_idx < prefix_len
 *                      FLEXATTN_PRIM_DOCUMENT  doc[q_idx] == doc[kv_idx]
 *                    A term with no bits is noop_mask (every pair). The
 *                    primitives share the parameters below.
 */
typedef enum {
  FLEXATTN_MASK_NOOP = 0,
  FLEXATTN_MASK_CAUSAL = 1,
  FLEXATTN_MASK_SLIDING_SINK = 2,
  FLEXATTN_MASK_DOCUMENT_CAUSAL = 3,
  FLEXATTN_MASK_PREFIX_LM = 4,
  FLEXATTN_MASK_COMPOSITE = 5
} flexattn_mask_kind;

enum {
  FLEXATTN_PRIM_CAUSAL = 1,
  FLEXATTN_PRIM_WINDOW = 2,
  FLEXATTN_PRIM_SINK = 4,
  FLEXATTN_PRIM_PREFIX = 8,
  FLEXATTN_PRIM_DOCUMENT = 16
};

typedef struct {
  int32_t window;          /* SLIDING_SINK: >= 1                                  */
  int32_t num_sinks;       /* SLIDING_SINK: >= 0                                  */
  const int32_t* doc_ids;  /* DOCUMENT_CAUSAL: device int32 [doc_batch][doc_len];
                              read through both q_idx and kv_idx; any id values */
  int32_t doc_batch;       /* DOCUMENT_CAUSAL: 1 (shared by all batches) or B     */
  int32_t doc_len;         /* DOCUMENT_CAUSAL: >= max(Q_LEN, KV_LEN)              */
  int32_t prefix_len;      /* PREFIX_LM: >= 0                                     */
  int32_t num_terms;       /* COMPOSITE: 1..4                                     */
  int32_t terms[4];        /* COMPOSITE: FLEXATTN_PRIM_* bit set of each term;
                              a primitive used by a term needs its parameter
                              (window >= 1, num_sinks >= 0, prefix_len >= 0,
                              doc_ids as for DOCUMENT_CAUSAL)               */
} flexattn_mask_params;

/*
 * score_mod kinds: s is the scaled score scale * (q . k); the modified score
 * replaces it before the softmax (page "attention-gym: examples, masks and
 * kernels for FlexAttention", section "A gallery that grew into a toolkit").
 *   NONE            s.
 *   ALIBI           s + m_h * (kv_idx - q_idx) (page "transformerlab",
 *                   section "Attention variants", row alibi).
 *   SOFTCAP         softcap * tanh(s / softcap) (page "Attention Backends",
 *                   tanh soft-capping).
 *   SOFTCAP_ALIBI   softcap * tanh(s / softcap) + m_h * (kv_idx - q_idx).
 * m_h is alibi_slopes[h] for query head h, or 2^(-8 (h + 1) / Hq) when
 * alibi_slopes is NULL.
 */
typedef enum {
  FLEXATTN_SCORE_NONE = 0,
  FLEXATTN_SCORE_ALIBI = 1,
  FLEXATTN_SCORE_SOFTCAP = 2,
  FLEXATTN_SCORE_SOFTCAP_ALIBI = 3
} flexattn_score_kind;

typedef struct {
  float softcap;              /* SOFTCAP kinds: > 0, finite                */
  const float* alibi_slopes;  /* ALIBI kinds: device float [Hq], or NULL   */
} flexattn_score_params;

typedef enum { FLEXATTN_F32 = 0, FLEXATTN_BF16 = 1, FLEXATTN_F16 = 2 } flexattn_dtype;

/*
 * A 4-D attention tensor [B][H][L][D] in device memory. stride[] are element
 * strides of the B, H, L and D dimensions; stride[3] must be 1 (rows
 * contiguous), each row must start 16-byte aligned (data and the other
 * strides times the element size are multiples of 16 bytes).
 */
typedef struct {
  void* data;
  flexattn_dtype dtype;
  int32_t B, H, L, D;
  int64_t stride[4];
} flexattn_tensor;

/*
 * BlockMask (page "tensorplay.nn.attention API", section BlockMask): the
 * element mask reduced to BLOCK_SIZE x BLOCK_SIZE tiles. A tile is empty when
 * every element in it is masked and is then never computed ("Basics"); a tile
 * is full when all BLOCK_SIZE^2 elements exist and are allowed, so the kernel
 * skips mask_mod on it ("Details", item 2); other non-empty tiles are partial.
 * For each (b, h, q row-tile) the partial tiles are listed in (kv_num_blocks,
 * kv_indices) and the full ones in (full_kv_num_blocks, full_kv_indices):
 * a count plus the KV tile positions, ascending, the unused tail set to 0.
 * Out-of-range elements of a tail tile count as masked, so a tail tile is
 * never full.
 *
 * Fields (all index tensors are caller-allocated device int32 buffers):
 *   B, H                 extents of the index tensors over batch and query
 *                        heads; 1 broadcasts over that dimension.
 *   Q_LEN, KV_LEN        sequence lengths; BLOCK_SIZE: the square tile edge,
 *                        128, 256, 384 or 512 (the page's default is 128;
 *                        from_kv_blocks takes 128 only).
 *   num_q_blocks (NQB)   ceil(Q_LEN / BLOCK_SIZE); num_kv_blocks (NKB) likewise.
 *   kv_num_blocks        [B][H][NQB]
 *   kv_indices           [B][H][NQB][NKB]
 *   full_kv_num_blocks   [B][H][NQB]
 *   full_kv_indices      [B][H][NQB][NKB]
 *   schedule             [B*H*NQB]: row ids (b*H + h)*NQB + qb ordered by
 *                        descending tile count (partial + full), ties by
 *                        ascending row id; the forward visits rows in this
 *                        order (longest first) for load balance.
 *   mask_kind, mask_params  the mask_mod the partial tiles are evaluated with.
 *   q_num_blocks, q_indices, full_q_num_blocks, full_q_indices
 *                        optional lists for the backward ("Details", items 3
 *                        and 4): for each (b, h, KV tile) the query tiles whose
 *                        tile is partial (resp. full), ascending, tail 0;
 *                        [B][H][NKB] counts and [B][H][NKB][NQB] indices.
 *                        flexattn_create_block_mask fills them when all four
 *                        pointers are non-NULL; NULL leaves them unbuilt (the
 *                        forward never reads them, flexattn_bwd needs them).
 * A caller may fill the struct from its own index lists (the from_kv_blocks
 * use); their contents are then trusted as given.
 */
typedef struct {
  int32_t B, H;
  int32_t Q_LEN, KV_LEN, BLOCK_SIZE;
  int32_t num_q_blocks, num_kv_blocks;
  int32_t* kv_num_blocks;
  int32_t* kv_indices;
  int32_t* full_kv_num_blocks;
  int32_t* full_kv_indices;
  int32_t* schedule;
  flexattn_mask_kind mask_kind;
  flexattn_mask_params mask_params;
  int32_t* q_num_blocks;
  int32_t* q_indices;
  int32_t* full_q_num_blocks;
  int32_t* full_q_indices;
  /* Q_BLOCK_SIZE of non-square tiles (the page's BLOCK_SIZE tuple
     (KV_BLOCK_SIZE, Q_BLOCK_SIZE), with BLOCK_SIZE the KV one): 0 means
     square tiles (= BLOCK_SIZE); else 128, 256, 384 or 512. An input to
     flexattn_create_block_mask, which writes the value it used. */
  int32_t Q_BLOCK_SIZE;
} flexattn_block_mask;

/*
 * Element counts of the BlockMask buffers for a build at (B, H, Q_LEN,
 * KV_LEN, block): num_elems for each of kv_num_blocks / full_kv_num_blocks,
 * idx_elems for each of kv_indices / full_kv_indices, sched_elems for
 * schedule. Host only. Output pointers must be non-NULL.
 */
/* The same for non-square tiles: kv_block x q_block. */
flexattn_status flexattn_block_mask_sizes_2d(int32_t B, int32_t H, int32_t Q_LEN, int32_t KV_LEN,
                                             int32_t kv_block, int32_t q_block,
                                             size_t* num_elems, size_t* idx_elems,
                                             size_t* sched_elems);
flexattn_status flexattn_block_mask_sizes(int32_t B, int32_t H, int32_t Q_LEN, int32_t KV_LEN,
                                          int32_t block, size_t* num_elems, size_t* idx_elems,
                                          size_t* sched_elems);

/*
 * create_block_mask (page "tensorplay.nn.attention API", section
 * create_block_mask): evaluates the mask_mod of `kind` over every
 * (b, h, q_idx, kv_idx), classifies each tile and writes the four index
 * tensors plus the schedule into the buffers `bm` points to.
 * separate_full_blocks != 0 lists full tiles apart from partial ones, so the
 * forward skips mask_mod on them; 0 lists every non-empty tile as partial
 * (full counts 0, full lists all 0) and mask_mod then runs on every tile, as
 * that page's create_block_mask parameter of the same name describes.
 * B and H give the extents to build (1 = one build broadcast over that
 * dimension; the enumerated kinds do not depend on b or h except through
 * per-batch doc_ids). On input the caller sets bm->kv_num_blocks,
 * kv_indices, full_kv_num_blocks, full_kv_indices and schedule; the call
 * fills every other field. block is the BLOCK_SIZE: 128, 256, 384 or 512
 * (UNSUPPORTED otherwise; size the buffers with the same block through
 * flexattn_block_mask_sizes). Asynchronous on `stream`.
 */
flexattn_status flexattn_create_block_mask(flexattn_mask_kind kind,
                                           const flexattn_mask_params* params, int32_t B,
                                           int32_t H, int32_t Q_LEN, int32_t KV_LEN,
                                           int32_t block, int32_t separate_full_blocks,
                                           flexattn_block_mask* bm, void* stream);

/*
 * The block-sparse attention forward (page "tensorplay.nn.attention API",
 * BlockMask "Details" item 1: the forward reduces along the KV dimension
 * using the per-row tile lists; item 2: mask_mod is skipped on full tiles;
 * page "FlagAttention", section "Operator overview": q [B,Hq,M,D], k/v
 * [B,Hkv,N,D], MQA/GQA). For every query row it visits only the listed KV
 * tiles, computes s = scale * q.k, applies the score_mod, applies the
 * mask_mod on partial tiles only, and accumulates the softmax-weighted sum of
 * V online, never materialising the score matrix.
 *   q     [B][Hq][Q_LEN][D]; k, v [B][Hkv][KV_LEN][D]; same dtype (F32,
 *         BF16 or F16); D in {64, 128}, or 256 for BF16 / F16; Hq a multiple
 *         of Hkv; query head h reads KV
 *         head h / (Hq / Hkv).
 *   bm    a BlockMask with bm->Q_LEN == Q_LEN, bm->KV_LEN == KV_LEN,
 *         bm->B in {1, B}, bm->H in {1, Hq}, BLOCK_SIZE (and Q_BLOCK_SIZE)
 *         128, 256, 384 or 512 (the kernels walk 128 x 128 pieces of larger
 *         tiles).
 *   out   [B][Hq][Q_LEN][D], same dtype as q (written).
 *   lse   device float [B][Hq][Q_LEN], contiguous (written): natural-log
 *         log-sum-exp of the modified, masked scores of each row.
 * A row with no allowed key gets out = 0 and lse = -inf. bf16 (fp16) inputs
 * are contracted on bf16 (fp16) MFMA with fp32 accumulation (softmax
 * probabilities are rounded to the input type for the P.V product); fp32
 * inputs are computed in fp32 throughout. BF16 / F16 limits
 * (FLEXATTN_ERR_UNSUPPORTED beyond them): k and v
 * row strides (stride[2]) at most 2^22 elements, and the per-row tile list
 * (num_kv_blocks ints) must fit in LDS beside the K/V staging buffers.
 * Work split (16-bit): one query head per workgroup, except that short query
 * tiles (Q_LEN <= 64, BlockMask broadcast over heads) pack several query
 * heads of one KV group into a workgroup; flexattn_fwd_make_plan reports the
 * packing a call gets. The split depends only on the shapes and the
 * BlockMask's extents; nothing else (no environment variable) selects it.
 * Asynchronous on `stream`.
 */
flexattn_status flexattn_fwd(const flexattn_tensor* q, const flexattn_tensor* k,
                             const flexattn_tensor* v, const flexattn_block_mask* bm,
                             flexattn_score_kind score_kind, const flexattn_score_params* params,
                             float scale, flexattn_tensor* out, float* lse, void* stream);

/*
 * Launch plan of the forward for given shapes (host only; reads no device
 * memory). It is the rule flexattn_fwd, flexattn_fwd_splitkv and
 * flexattn_fwd_paged apply, reported so that a caller can size a split-KV
 * call without restating it:
 *   waves_per_head       4: one 128-row query tile per workgroup; 2 or 1:
 *                        short query tiles, several heads per workgroup.
 *   heads_per_workgroup  query heads of one KV group sharing a workgroup and
 *                        its K/V stream (4 / waves_per_head).
 *   row16                1 when the 16-row MFMA step runs (at most 16 query
 *                        rows per head, one wave per head).
 *   work_items           workgroups of one unsplit launch.
 *   num_splits           KV slices per item that fill target_workgroups
 *                        once when items are few (1 = do not split): at most
 *                        num_kv_blocks and 64.
 * Shapes: q [B][Hq][Q_LEN][D], KV heads Hkv, dtype as flexattn_tensor's;
 * bm: the BlockMask of the call (its extents, tile counts and block sizes
 * are read; its device buffers are not). target_workgroups <= 0 means 512
 * (two workgroups on each of 256 CUs). fp32 calls get waves_per_head 0,
 * heads_per_workgroup 1, row16 0, num_splits 1 (the fp32 path does not
 * split) and the fp32 kernel's workgroup count (one per 8 query rows).
 * Errors: INVALID_ARG for NULL pointers, non-positive shapes or a BlockMask
 * that does not match them; UNSUPPORTED for other dtypes or block sizes.
 */
typedef struct {
  int32_t waves_per_head;
  int32_t heads_per_workgroup;
  int32_t row16;
  int32_t num_splits;
  int64_t work_items;
} flexattn_fwd_plan;

flexattn_status flexattn_fwd_make_plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t Q_LEN,
                                       int32_t D, flexattn_dtype dtype,
                                       const flexattn_block_mask* bm, int32_t target_workgroups,
                                       flexattn_fwd_plan* plan);

/*
 * Split-KV forward for calls with few query tiles and long KV lists (decode
 * and short prefills): each query tile's KV tile list is cut into
 * num_splits contiguous slices, one workgroup each, so the launch fills the
 * chip; each slice writes its normalised O and its LSE in fp32 to
 * `workspace`, and a combine pass merges them (LSE = ln sum exp LSE_s,
 * O = sum exp(LSE_s - LSE) O_s), which is the online softmax's rescaling
 * applied across slices. Same method and outputs as flexattn_fwd (section
 * "Details" of page "tensorplay.nn.attention API", items 1 and 2), bf16 and
 * fp16 (UNSUPPORTED for fp32), 1 <= num_splits <= 256; num_splits = 1 is
 * flexattn_fwd. workspace: device memory of at least
 * flexattn_fwd_splitkv_workspace_bytes(B, Hq, Q_LEN, D, num_splits) bytes,
 * 16-byte aligned, caller-allocated and overwritten. Asynchronous on
 * `stream`.
 */
size_t flexattn_fwd_splitkv_workspace_bytes(int32_t B, int32_t Hq, int32_t Q_LEN, int32_t D,
                                            int32_t num_splits);
flexattn_status flexattn_fwd_splitkv(const flexattn_tensor* q, const flexattn_tensor* k,
                                     const flexattn_tensor* v, const flexattn_block_mask* bm,
                                     flexattn_score_kind score_kind,
                                     const flexattn_score_params* params, float scale,
                                     int32_t num_splits, void* workspace, size_t workspace_bytes,
                                     flexattn_tensor* out, float* lse, void* stream);

/*
 * flexattn_fwd_splitkv without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The slices' fp32 partials go to a
 * scratch array inside the library: one copy of FLEXATTN_SCRATCH_BYTES
 * (32 MiB) per GPU, held until the process ends; the first call on a device
 * looks up its address there (no allocation). The call allocates nothing
 * and frees nothing. Same arguments, method and outputs as
 * flexattn_fwd_splitkv minus the workspace; num_splits = 1 runs flexattn_fwd.
 * INVALID_ARG when the partials need more than the scratch holds
 * (flexattn_fwd_splitkv_workspace_bytes(B, Hq, Q_LEN, D, num_splits) >
 * FLEXATTN_SCRATCH_BYTES) or when `stream` belongs to another device than
 * the current one. Every call on one GPU shares its scratch, which keeps the
 * last call's contents: calls that overlap in time on one GPU (several
 * streams, several host threads) race and must be ordered by the caller.
 */
#define FLEXATTN_SCRATCH_BYTES (32u * 1024u * 1024u)
flexattn_status flexattn_fwd_splitkv_noalloc(const flexattn_tensor* q, const flexattn_tensor* k,
                                             const flexattn_tensor* v,
                                             const flexattn_block_mask* bm,
                                             flexattn_score_kind score_kind,
                                             const flexattn_score_params* params, float scale,
                                             int32_t num_splits, flexattn_tensor* out, float* lse,
                                             void* stream);

/*
 * Paged KV cache (page "FlagAttention", operator overview: paged attention,
 * queries over a KV cache kept in fixed-size pages). The cache holds
 * num_pages pages of page_size key rows per KV head; a sequence's keys are
 * laid out page by page through its row of the page table.
 * page_table: device int32 [B][max_pages]; entry (b, p) is the cache page
 * that holds keys [p * page_size, (p + 1) * page_size) of batch b. Entries
 * past the pages KV_LEN needs are not read. An entry outside
 * [0, num_pages) is clamped into it (wrong output, no out-of-bounds read).
 */
typedef struct {
  const int32_t* page_table;
  int32_t max_pages;  /* entries per batch row; max_pages * page_size >= KV_LEN */
} flexattn_page_table;

/*
 * Forward over a paged KV cache: the same method and outputs as
 * flexattn_fwd (and, with num_splits > 1, flexattn_fwd_splitkv, whose
 * workspace rules apply) with keys read through the page table. k_cache and
 * v_cache are flexattn_tensors with B = num_pages, H = Hkv, L = page_size
 * (a multiple of 128, so a BlockMask tile never straddles pages), any
 * 16-byte-multiple strides. The sequence length is bm->KV_LEN. bf16 or
 * fp16 (UNSUPPORTED otherwise); page sizes that are not multiples of 128 are
 * UNSUPPORTED. Asynchronous on `stream`.
 */
flexattn_status flexattn_fwd_paged(const flexattn_tensor* q, const flexattn_tensor* k_cache,
                                   const flexattn_tensor* v_cache,
                                   const flexattn_page_table* pages,
                                   const flexattn_block_mask* bm, flexattn_score_kind score_kind,
                                   const flexattn_score_params* params, float scale,
                                   int32_t num_splits, void* workspace, size_t workspace_bytes,
                                   flexattn_tensor* out, float* lse, void* stream);

/*
 * from_kv_blocks (page "tensorplay.nn.attention API", BlockMask.from_kv_blocks):
 * completes a BlockMask whose tile lists the caller filled. On input the
 * caller sets every field of `bm`: the extents, lengths, BLOCK_SIZE (128),
 * num_q_blocks / num_kv_blocks, mask_kind / mask_params (the mask the
 * partial tiles are evaluated with; NOOP makes every listed tile dense),
 * the four list buffers (full counts may be all 0) and schedule; the q_*
 * buffers are optional as in flexattn_create_block_mask. The call writes
 * the schedule and, when the q_* buffers are set, the backward lists.
 * It also checks the lists on the GPU and writes *status (device int32):
 * 0 when they are valid, else the OR of 1 (a count outside [0, NKB]),
 * 2 (an index outside [0, NKB)), 4 (a list not strictly ascending),
 * 8 (a tile in both the partial and the full list of a row) and 16 (a full
 * tile not entirely inside Q_LEN x KV_LEN: all BLOCK_SIZE^2 elements of a
 * full tile are allowed, so a tail tile can only be partial). The schedule
 * and backward lists of invalid lists are meaningless; read *status before
 * using the BlockMask. Host-side argument errors return as for
 * flexattn_create_block_mask. Asynchronous on `stream`.
 */
flexattn_status flexattn_block_mask_from_kv_blocks(flexattn_block_mask* bm, int32_t* status,
                                                   void* stream);

/*
 * Backward of flexattn_fwd: the gradients of the forward's output with
 * respect to q, k and v for an upstream gradient d_out (page
 * "tensorplay.nn.attention API", section BlockMask, "Details": dQ walks each
 * query tile's KV tiles from items 1 and 2; dK and dV walk each KV tile's
 * query tiles from items 3 and 4, so `bm` must carry q_num_blocks,
 * q_indices, full_q_num_blocks and full_q_indices). mask_mod runs on partial
 * tiles only, as in the forward.
 *   q, k, v, score_kind, params, scale: exactly as given to flexattn_fwd.
 *   lse   the forward's LSE, device float [B][Hq][Q_LEN], contiguous.
 *   d_out dL/dO, shaped like the forward's output [B][Hq][Q_LEN][D].
 *   dq    written: dL/dq, shaped like q.
 *   dk,dv written: dL/dk, dL/dv [B][Hkv][KV_LEN][D]; each sums the query heads
 *         of its GQA group (in a fixed order: the result is deterministic).
 *   workspace  device float [B * Hq * Q_LEN], caller-allocated and
 *         overwritten with Delta_i = sum_j P_ij dP_ij, which equals dO_i . O_i
 *         but is formed from fp32 P and dP, so the forward's output is not an
 *         input.
 * All seven tensors share one dtype, BF16 or F16 (q of another dtype is
 * UNSUPPORTED, a tensor differing from q INVALID_ARG); D in {64, 128}
 * (UNSUPPORTED otherwise). The products run on the matching MFMA with fp32
 * accumulation; P and dS are rounded to the input type for the second
 * products and the gradients are stored in it. Strides and alignment as for
 * flexattn_fwd; a row stride (stride[2]) of q, k, v or d_out above 2^22
 * elements is UNSUPPORTED (the kernels address a tile of up to 128 rows with
 * 32-bit offsets). Rows with no allowed key (LSE = -inf) get dq = 0.
 * Asynchronous on `stream`; no host synchronisation.
 */
flexattn_status flexattn_bwd(const flexattn_tensor* q, const flexattn_tensor* k,
                             const flexattn_tensor* v, const float* lse,
                             const flexattn_tensor* d_out,
                             const flexattn_block_mask* bm, flexattn_score_kind score_kind,
                             const flexattn_score_params* params, float scale,
                             flexattn_tensor* dq, flexattn_tensor* dk, flexattn_tensor* dv,
                             float* workspace, void* stream);

/*
 * Training pair (the backward's row sums Delta_i = sum_j P_ij dP_ij equal
 * dO_i . O_i, since O_i = sum_j P_ij v_j; the chain rule of the same
 * forward as flexattn_bwd). flexattn_fwd_train is flexattn_fwd (16-bit
 * inputs, no split, contiguous K/V) that also writes O in fp32 to out_f32,
 * device float [B][Hq][Q_LEN][D] contiguous, 16-byte aligned, caller-
 * allocated. flexattn_bwd_from_out is flexattn_bwd with Delta taken as
 * dO . out_f32 in one pass over them instead of recomputing P and dP for
 * it; out_f32 must come from flexattn_fwd_train on the same inputs (fp32
 * O keeps Delta within the gradients' error bound, the rounded 16-bit O
 * does not). Same errors as the calls they extend, plus INVALID_ARG for a
 * NULL or misaligned out_f32. Asynchronous on `stream`.
 */
flexattn_status flexattn_fwd_train(const flexattn_tensor* q, const flexattn_tensor* k,
                                   const flexattn_tensor* v, const flexattn_block_mask* bm,
                                   flexattn_score_kind score_kind,
                                   const flexattn_score_params* params, float scale,
                                   flexattn_tensor* out, float* lse, float* out_f32,
                                   void* stream);
flexattn_status flexattn_bwd_from_out(const flexattn_tensor* q, const flexattn_tensor* k,
                                      const flexattn_tensor* v, const float* lse,
                                      const float* out_f32, const flexattn_tensor* d_out,
                                      const flexattn_block_mask* bm,
                                      flexattn_score_kind score_kind,
                                      const flexattn_score_params* params, float scale,
                                      flexattn_tensor* dq, flexattn_tensor* dk,
                                      flexattn_tensor* dv, float* workspace, void* stream);

/* Message of the last failed call on this thread ("" if none). Host only. */
const char* flexattn_last_error(void);

/* Library version string. Host only. */
const char* flexattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLEXATTN_H */
