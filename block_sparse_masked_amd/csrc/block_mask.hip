// BlockMask builder for gfx950: classify every 128x128 tile of the element
// mask as empty / partial / full, write the ascending per-row tile lists,
// then order the rows by tile count for the forward's work schedule.
//
// Follows page "tensorplay.nn.attention API", section create_block_mask
// (separate_full_blocks=True) and section BlockMask ("Basics": a tile is
// skipped only when all its elements are masked; "Details" item 2: full tiles
// listed apart; the row-compressed count + index-list format).
//
// Counting. For the enumerated mask kinds the allowed keys of one query row
// form at most two intervals, so the allowed count of a row inside a KV tile
// is O(1) arithmetic and a tile's count is a sum over its 128 rows:
//   NOOP          [0, KV_LEN)
//   CAUSAL        [0, q]
//   SLIDING_SINK  [q - window + 1, q]  union  [0, min(sinks - 1, q)]
//   DOCUMENT      [start of q's run of equal ids, q]  -- valid when the ids
//                 never decrease (each document one contiguous run, the packed
//                 layout); otherwise every element is compared.
// The counts are exact, so the classification equals a per-element
// evaluation of the mask.
#include "common.hpp"
#include "launch.hpp"

namespace fa {

namespace {

constexpr int kRowThreads = kBlock;  // one thread per query row of a tile

struct BuildArgs {
  int kind;
  MaskParams mp;
  int doc_len;
  const int* sorted_flags;  // document kind: per-chunk sortedness (schedule buffer)
  int Bm, Hm, Q_LEN, KV_LEN, NQB, NKB;
  int BS;   // KV_BLOCK_SIZE: a multiple of 128
  int QBS;  // Q_BLOCK_SIZE: a multiple of 128 (rows are counted 128 at a time)
  int* kv_num;
  int* kv_idx;
  int* full_num;
  int* full_idx;
  int separate_full;  // 0: full tiles are listed with the partial ones
};

__device__ __forceinline__ int clamp_len(int lo, int hi) { return hi >= lo ? hi - lo + 1 : 0; }

// Wave-wide sum (64 lanes) with cross-lane shuffles.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Inclusive prefix sum over the 128 threads of the block (2 waves).
__device__ __forceinline__ int block_incl_scan128(int v, int* lds2) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) lds2[wave] = v;
  __syncthreads();
  if (wave == 1) v += lds2[0];
  __syncthreads();
  return v;
}

// Inclusive max-scan over the 128 threads (2 waves).
__device__ __forceinline__ int block_incl_max128(int v, int* lds2) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int u = __shfl_up(v, off, 64);
    if (lane >= off) v = max(v, u);
  }
  if (lane == 63) lds2[wave] = v;
  __syncthreads();
  if (wave == 1) v = max(v, lds2[0]);
  __syncthreads();
  return v;
}

// First index of the run containing position q0 in a non-decreasing doc row:
// the smallest i with doc[i] == doc[q0]. Two rounds of a 128-way parallel
// search over [0, q0].
__device__ int run_start_of(const int* doc, int q0, int* lds) {
  const int t = threadIdx.x;
  const int key = doc[q0];
  // First pass: coarse grid of 128 probes over [0, q0].
  const int step = (q0 + kRowThreads) / kRowThreads;  // >= 1, covers [0, q0]
  int p = t * step;
  int hit = (p <= q0 && doc[p] < key) ? t : -1;  // last probe strictly before the run
  hit = block_incl_max128(hit, lds);
  if (t == kRowThreads - 1) lds[2] = hit;  // inclusive scan: thread 127 holds the max
  __syncthreads();
  const int lastp = lds[2];
  __syncthreads();
  if (lastp < 0) return 0;  // probe 0 (position 0) already holds the key
  int lo, hi;
  lo = lastp * step + 1;             // first candidate after the last "before" probe
  hi = min(q0, lo + step - 1);        // the run starts within [lo, hi]
  // Second pass: positions lo + t*r covering [lo, hi] with r = ceil(len/128).
  const int len = hi - lo + 1;
  const int r = (len + kRowThreads - 1) / kRowThreads;
  int first = 0x7fffffff;
  for (int i = 0; i < r; ++i) {
    int pos = lo + t * r + i;
    if (pos <= hi && doc[pos] == key) first = min(first, pos);
  }
  // block min via negated max-scan
  int neg = block_incl_max128(-first, lds);
  if (threadIdx.x == 127) lds[2] = -neg;
  __syncthreads();
  int res = lds[2];
  __syncthreads();
  return res;
}

// Run [first, last] of value doc[q] in a non-decreasing id row of n entries
// (binary searches for the first entry >= and the first entry > the value).
__device__ __forceinline__ void doc_run_of(const int* doc, int n, int q, int& first, int& last) {
  const int v = doc[q];
  int lo = 0, hi = q;  // first index with doc >= v lies in [0, q]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (doc[mid] < v) lo = mid + 1; else hi = mid;
  }
  first = lo;
  lo = q;
  hi = n - 1;  // last index with doc <= v lies in [q, n - 1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (doc[mid] > v) hi = mid - 1; else lo = mid;
  }
  last = lo;
}

// Sortedness of the document ids, in NQB chunks per document row: workgroup
// (r, c) checks that doc row r never decreases across positions
// [c * chunk, (c + 1) * chunk] and writes 1 (sorted) or 0 to flags[r * NQB + c].
// The flags live in the schedule buffer, which the schedule kernel overwrites
// after the classify kernel has read them.
__global__ __launch_bounds__(256) void doc_sorted_kernel(const int* doc, long long bstride, int n,
                                                         int chunk, int nqb, int* flags) {
  const int r = blockIdx.y, c = blockIdx.x;
  const int* row = doc + r * bstride;
  const int lo = c * chunk;
  const int hi = min(n - 1, lo + chunk);  // last pair checked: (hi - 1, hi)
  int bad = 0;
  for (int i = lo + threadIdx.x; i < hi; i += 256) bad |= (row[i] > row[i + 1]);
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) flags[r * nqb + c] = bad ? 0 : 1;
}

// Adds the allowed count of the key interval [lo, hi] of one query row to the
// per-tile totals: the two end tiles directly, the tiles in between (every
// key allowed) through the difference array `dif` (prefix-summed later).
__device__ __forceinline__ void add_interval(int* tot, int* dif, int lo, int hi, int sign, int bs) {
  if (hi < lo) return;
  const int jl = lo / bs, jh = hi / bs;
  if (jl == jh) {
    atomicAdd(&tot[jl], sign * (hi - lo + 1));
    return;
  }
  atomicAdd(&tot[jl], sign * ((jl + 1) * bs - lo));
  atomicAdd(&tot[jh], sign * (hi - jh * bs + 1));
  if (jh > jl + 1) {
    atomicAdd(&dif[jl + 1], sign * bs);
    atomicAdd(&dif[jh], -sign * bs);
  }
}

template <int KIND>
__global__ __launch_bounds__(kRowThreads) void classify_kernel(BuildArgs a) {
  extern __shared__ int smem[];  // tot[NKB], dif[NKB + 1]
  __shared__ int scratch[4];
  const int row = blockIdx.x;  // (bm * Hm + hm) * NQB + qb
  const int qb = row % a.NQB;
  const int bm = row / (a.NQB * a.Hm);
  const int t = threadIdx.x;
  const int NKB = a.NKB;
  const int BS = a.BS, QBS = a.QBS;
  int* tot = smem;
  int* dif = smem + NKB;
  for (int j = t; j < 2 * NKB + 1; j += kRowThreads) smem[j] = 0;

  // The tile row's BS query rows, 128 at a time (one per thread); each
  // query row's allowed keys are counted into the per-tile totals.
  for (int sb = 0; sb < QBS / kBlock; ++sb) {
  const int q = qb * QBS + sb * kBlock + t;
  const bool qvalid = q < a.Q_LEN;
  // Per-row allowed intervals: I1 = [lo1, hi1], I2 = [lo2, hi2] (may be empty).
  int lo1 = 0, hi1 = -1, lo2 = 0, hi2 = -1;
  bool brute = false;
  const int* doc = nullptr;
  // COMPOSITE: each term's allowed keys form one interval (its interval
  // primitives, intersected with the query's document run when the term
  // tests documents); the union of the terms' intervals is counted exactly
  int clo[kMaxTerms], chi[kMaxTerms];
  int nint = 0;
  if constexpr (KIND == MASK_COMPOSITE) {
    bool uses_doc = false;
    for (int tt = 0; tt < a.mp.nterms; ++tt) uses_doc |= (a.mp.terms[tt] & PRIM_DOCUMENT) != 0;
    int run_lo = 0, run_hi = a.KV_LEN - 1;
    if (uses_doc) {
      const int drow = a.mp.doc_bstride > 0 ? bm : 0;
      doc = a.mp.doc + (long long)drow * a.mp.doc_bstride;
      int bad = 0;
      for (int c = t; c < a.NQB; c += kRowThreads) bad |= (a.sorted_flags[drow * a.NQB + c] == 0);
      brute = __syncthreads_or(bad) != 0;
      if (!brute && qvalid) doc_run_of(doc, max(a.Q_LEN, a.KV_LEN), q, run_lo, run_hi);
    }
    for (int tt = 0; tt < a.mp.nterms; ++tt) {
      const int bits = a.mp.terms[tt];
      int lo, hi;
      term_interval(bits, q, a.mp, lo, hi);
      if (bits & PRIM_DOCUMENT) {
        lo = max(lo, run_lo);
        hi = min(hi, run_hi);
      }
      lo = max(lo, 0);
      hi = min(hi, a.KV_LEN - 1);
      if (lo > hi) continue;
      // insert in ascending order of lo
      int i = nint++;
      while (i > 0 && clo[i - 1] > lo) {
        clo[i] = clo[i - 1];
        chi[i] = chi[i - 1];
        --i;
      }
      clo[i] = lo;
      chi[i] = hi;
    }
  } else if constexpr (KIND == MASK_DOCUMENT) {
    const int drow = a.mp.doc_bstride > 0 ? bm : 0;
    doc = a.mp.doc + (long long)drow * a.mp.doc_bstride;
    // sorted unless a chunk flag of this document row says otherwise
    int bad = 0;
    for (int c = t; c < a.NQB; c += kRowThreads) bad |= (a.sorted_flags[drow * a.NQB + c] == 0);
    const bool sorted = __syncthreads_or(bad) == 0;
    if (sorted) {
      const int q0 = qb * QBS + sb * kBlock;
      const int s0 = run_start_of(doc, min(q0, a.doc_len - 1), scratch);
      // run boundaries inside this tile, then the latest boundary <= q
      int bnd = (qvalid && q > q0 && doc[q] != doc[q - 1]) ? q : -1;
      bnd = block_incl_max128(bnd, scratch);
      const int start = bnd >= 0 ? bnd : s0;
      lo1 = start;
      hi1 = q;
    } else {
      brute = true;
    }
  } else if constexpr (KIND == MASK_NOOP) {
    lo1 = 0;
    hi1 = a.KV_LEN - 1;
  } else if constexpr (KIND == MASK_CAUSAL) {
    lo1 = 0;
    hi1 = q;
  } else if constexpr (KIND == MASK_PREFIX_LM) {
    // [0, q] u [0, prefix - 1] is one interval
    lo1 = 0;
    hi1 = max(q, a.mp.prefix - 1);
  } else {  // SLIDING_SINK
    lo1 = max(0, q - a.mp.window + 1);
    hi1 = q;
    lo2 = 0;
    hi2 = min(a.mp.sinks - 1, q);
  }
  hi1 = min(hi1, a.KV_LEN - 1);
  hi2 = min(hi2, a.KV_LEN - 1);
  __syncthreads();  // totals zeroed (first pass), scratch free

  if (qvalid) {
    if (KIND == MASK_COMPOSITE && brute) {
      // unsorted ids: evaluate every key of the row
      const int dq = doc[q];
      for (int j = 0; j < NKB; ++j) {
        int cnt = 0;
        const int c1 = min(j * BS + BS, a.KV_LEN);
        for (int kv = j * BS; kv < c1; ++kv) cnt += composite_allowed(a.mp, q, kv, dq, doc[kv]);
        if (cnt) atomicAdd(&tot[j], cnt);
      }
    } else if (KIND == MASK_COMPOSITE) {
      // merge the sorted intervals into disjoint ones and count each once
      int i = 0;
      while (i < nint) {
        int lo = clo[i], hi = chi[i];
        ++i;
        while (i < nint && clo[i] <= hi + 1) hi = max(hi, chi[i++]);
        add_interval(tot, dif, lo, hi, 1, BS);
      }
    } else if (KIND == MASK_DOCUMENT && brute) {
      // unsorted ids: compare every key <= q with this row's id
      const int dq = doc[q];
      const int e = min(q, a.KV_LEN - 1);
      for (int j = 0; j * BS <= e; ++j) {
        int cnt = 0;
        const int c1 = min(j * BS + BS - 1, e);
        for (int kv = j * BS; kv <= c1; ++kv) cnt += (doc[kv] == dq);
        if (cnt) atomicAdd(&tot[j], cnt);
      }
    } else {
      add_interval(tot, dif, lo1, hi1, 1, BS);
      if constexpr (KIND == MASK_SLIDING_SINK) {
        // |I1 u I2| = |I1| + |I2| - |I1 n I2|
        add_interval(tot, dif, lo2, hi2, 1, BS);
        add_interval(tot, dif, max(lo1, lo2), min(hi1, hi2), -1, BS);
      }
    }
  }
  __syncthreads();
  }  // sub-blocks of the tile row

  // Totals (difference array prefix-summed in chunks of 128 tiles), then
  // classify and compact, keeping ascending order.
  const long long base = (long long)row * NKB;
  int np_total = 0, nf_total = 0, run = 0;
  for (int j0 = 0; j0 < NKB; j0 += kRowThreads) {
    const int j = j0 + t;
    const int d = j < NKB ? dif[j] : 0;
    const int incD = block_incl_scan128(d, scratch);
    int isP = 0, isF = 0;
    if (j < NKB) {
      const int cnt = tot[j] + run + incD;
      isF = a.separate_full && (cnt == QBS * BS);
      isP = (cnt > 0 && !isF);
    }
    const int incP = block_incl_scan128(isP, scratch);
    const int incF = block_incl_scan128(isF, scratch);
    if (isP) a.kv_idx[base + np_total + incP - 1] = j;
    if (isF) a.full_idx[base + nf_total + incF - 1] = j;
    // chunk totals live in the last thread
    if (t == kRowThreads - 1) {
      scratch[0] = incD;
      scratch[2] = incP;
      scratch[3] = incF;
    }
    __syncthreads();
    run += scratch[0];
    np_total += scratch[2];
    nf_total += scratch[3];
    __syncthreads();
  }
  // zero the unused tails
  for (int j = t; j < NKB; j += kRowThreads) {
    if (j >= np_total) a.kv_idx[base + j] = 0;
    if (j >= nf_total) a.full_idx[base + j] = 0;
  }
  if (t == 0) {
    a.kv_num[row] = np_total;
    a.full_num[row] = nf_total;
  }
}

// Stable ordering of rows by descending tile count (ties: ascending row id),
// one workgroup: histogram, suffix offsets (block scan), then a stable
// scatter in chunks of 1024 rows.
constexpr int kSchedThreads = 1024;

// Exclusive prefix sum over the 1024 threads of the block.
__device__ __forceinline__ int block_excl_scan1024(int v, int* lds16) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(x, off, 64);
    if (lane >= off) x += u;
  }
  if (lane == 63) lds16[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? lds16[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int u = __shfl_up(w, off, 64);
      if (lane >= off) w += u;
    }
    if (lane < 16) lds16[lane] = w;  // inclusive wave totals
  }
  __syncthreads();
  const int before = wave > 0 ? lds16[wave - 1] : 0;
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int* kv_num,
                                                                 const int* full_num, int n,
                                                                 int nbins, int* schedule) {
  extern __shared__ int sm[];
  int* hist = sm;             // [nbins]  -> bin offsets
  int* running = sm + nbins;  // [nbins]
  __shared__ __attribute__((aligned(16))) int keys[kSchedThreads];
  __shared__ int wtot[16];
  const int t = threadIdx.x;
  for (int c = t; c < nbins; c += kSchedThreads) {
    hist[c] = 0;
    running[c] = 0;
  }
  __syncthreads();
  // keys are clamped to the bins (caller-given lists may hold bad counts)
  for (int i = t; i < n; i += kSchedThreads)
    atomicAdd(&hist[min(max(kv_num[i] + full_num[i], 0), nbins - 1)], 1);
  __syncthreads();
  // offsets for descending keys: off[c] = sum_{c' > c} hist[c']. Thread t owns
  // the contiguous bins (hi_bin - seg, hi_bin], scanned from the top.
  const int seg = (nbins + kSchedThreads - 1) / kSchedThreads;
  const int hi_bin = nbins - 1 - t * seg;
  int local = 0;
  for (int s2 = 0; s2 < seg; ++s2) {
    const int c = hi_bin - s2;
    if (c >= 0) local += hist[c];
  }
  int acc = block_excl_scan1024(local, wtot);
  for (int s2 = 0; s2 < seg; ++s2) {
    const int c = hi_bin - s2;
    if (c >= 0) {
      const int h = hist[c];
      hist[c] = acc;  // becomes the offset of bin c
      acc += h;
    }
  }
  __syncthreads();
  for (int base = 0; base < n; base += kSchedThreads) {
    const int i = base + t;
    const int key = (i < n) ? min(max(kv_num[i] + full_num[i], 0), nbins - 1) : -1;
    keys[t] = key;
    __syncthreads();
    if (i < n) {
      // equal keys earlier in this chunk, four at a time
      int rank = 0;
      const int4* k4 = reinterpret_cast<const int4*>(keys);
      for (int u = 0; u < t / 4; ++u) {
        const int4 kk = k4[u];
        rank += (kk.x == key) + (kk.y == key) + (kk.z == key) + (kk.w == key);
      }
      for (int u = t & ~3; u < t; ++u) rank += (keys[u] == key);
      schedule[hist[key] + running[key] + rank] = i;
    }
    __syncthreads();
    if (i < n) atomicAdd(&running[key], 1);
    __syncthreads();
  }
}

// Backward lists ("Details", items 3 and 4): for BlockMask row group bh and
// KV tile j, the query tiles whose partial (full) list holds j, ascending.
// One workgroup per row group: the rows' lists are scattered into a class
// grid in LDS (one byte per tile, transposed: [NKB][NQB]), then each thread
// compacts one KV tile's column. Groups whose grid does not fit fall back to
// one thread per KV tile binary-searching every row's ascending lists.
constexpr int kTransposeThreads = 256;
constexpr int kTransposeLdsBytes = 48 * 1024;

__device__ __forceinline__ bool sorted_contains(const int* list, int n, int j) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int v = list[mid];
    if (v == j) return true;
    if (v < j) lo = mid + 1;
    else hi = mid;
  }
  return false;
}

__global__ __launch_bounds__(kTransposeThreads) void transpose_kernel(
    const int* kv_num, const int* kv_idx, const int* full_num, const int* full_idx, int NQB,
    int NKB, int* q_num, int* q_idx, int* fq_num, int* fq_idx) {
  __shared__ unsigned char cls[kTransposeLdsBytes];  // [NKB][NQB]: 0 empty, 1 partial, 2 full
  const int bh = blockIdx.x;
  const int t = threadIdx.x;
  const long long rows = (long long)bh * NQB;
  const bool in_lds = (long long)NQB * NKB <= kTransposeLdsBytes;
  if (in_lds) {
    for (int e = t; e < NQB * NKB; e += kTransposeThreads) cls[e] = 0;
    __syncthreads();
    // scatter: (row i, list slot u) pairs spread over the threads
    for (long long e = t; e < (long long)NQB * NKB; e += kTransposeThreads) {
      const int i = (int)(e / NKB), u = (int)(e % NKB);
      const long long r = rows + i;
      const int cp = min(max(kv_num[r], 0), NKB);
      const int cf = min(max(full_num[r], 0), NKB);
      if (u < cp) {
        const int j = kv_idx[r * NKB + u];
        if (j >= 0 && j < NKB) cls[j * NQB + i] = 1;
      }
      if (u < cf) {
        const int j = full_idx[r * NKB + u];
        if (j >= 0 && j < NKB) cls[j * NQB + i] = 2;
      }
    }
    __syncthreads();
  }
  for (int j = t; j < NKB; j += kTransposeThreads) {
    const long long out = ((long long)bh * NKB + j) * NQB;
    int np = 0, nf = 0;
    for (int i = 0; i < NQB; ++i) {
      int c;
      if (in_lds) {
        c = cls[j * NQB + i];
      } else {
        const long long r = rows + i;
        c = sorted_contains(full_idx + r * NKB, min(max(full_num[r], 0), NKB), j) ? 2
            : sorted_contains(kv_idx + r * NKB, min(max(kv_num[r], 0), NKB), j) ? 1 : 0;
      }
      if (c == 1) q_idx[out + np++] = i;
      if (c == 2) fq_idx[out + nf++] = i;
    }
    for (int u = np; u < NQB; ++u) q_idx[out + u] = 0;
    for (int u = nf; u < NQB; ++u) fq_idx[out + u] = 0;
    q_num[(long long)bh * NKB + j] = np;
    fq_num[(long long)bh * NKB + j] = nf;
  }
}

// Checks of caller-given lists (from_kv_blocks): one 128-thread workgroup per
// row. Flags OR-ed into *status: 1 a count outside [0, NKB]; 2 an index
// outside [0, NKB); 4 a list not strictly ascending; 8 a tile in both lists;
// 16 a full tile that is not entirely inside Q_LEN x KV_LEN (a full tile has
// all BLOCK_SIZE^2 elements allowed, so it cannot cross a sequence end).
__global__ void clear_status_kernel(int* status) { *status = 0; }

__global__ __launch_bounds__(kRowThreads) void validate_kernel(const int* kv_num, const int* kv_idx,
                                                             const int* full_num,
                                                             const int* full_idx, int NQB, int NKB,
                                                             int Q_LEN, int KV_LEN, int* status) {
  const long long row = blockIdx.x;
  const bool q_tail = (int)(row % NQB) * kBlock + kBlock > Q_LEN;
  const int t = threadIdx.x;
  const int np_raw = kv_num[row], nf_raw = full_num[row];
  int flags = 0;
  if (np_raw < 0 || np_raw > NKB || nf_raw < 0 || nf_raw > NKB) flags |= 1;
  const int np = min(max(np_raw, 0), NKB), nf = min(max(nf_raw, 0), NKB);
  const int* P = kv_idx + row * NKB;
  const int* F = full_idx + row * NKB;
  for (int u = t; u < np; u += kRowThreads) {
    const int j = P[u];
    if (j < 0 || j >= NKB) flags |= 2;
    if (u > 0 && P[u - 1] >= j) flags |= 4;
    if (sorted_contains(F, nf, j)) flags |= 8;
  }
  for (int u = t; u < nf; u += kRowThreads) {
    const int j = F[u];
    if (j < 0 || j >= NKB) flags |= 2;
    if (u > 0 && F[u - 1] >= j) flags |= 4;
    if (q_tail || j * kBlock + kBlock > KV_LEN) flags |= 16;
  }
  if (flags) atomicOr(status, flags);
}

}  // namespace

hipError_t launch_from_kv_blocks(const BuildLaunch& L, int* status, hipStream_t stream) {
  const int rows = L.Bm * L.Hm * L.NQB;
  clear_status_kernel<<<1, 1, 0, stream>>>(status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  validate_kernel<<<rows, kRowThreads, 0, stream>>>(L.kv_num, L.kv_idx, L.full_num, L.full_idx,
                                                    L.NQB, L.NKB, L.Q_LEN, L.KV_LEN, status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nbins = L.NKB + 1;
  schedule_kernel<<<1, kSchedThreads, sizeof(int) * 2 * (size_t)nbins, stream>>>(
      L.kv_num, L.full_num, rows, nbins, L.schedule);
  if (L.q_num) {
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    transpose_kernel<<<L.Bm * L.Hm, kTransposeThreads, 0, stream>>>(
        L.kv_num, L.kv_idx, L.full_num, L.full_idx, L.NQB, L.NKB, L.q_num, L.q_idx,
        L.full_q_num, L.full_q_idx);
  }
  return hipGetLastError();
}

int max_build_kv_blocks() {
  // 2*NKB+1 ints of dynamic LDS for the classify kernel, two int arrays of
  // NKB+1 bins for the schedule kernel; stay well inside 64 KiB.
  return 4096;
}

hipError_t launch_build(const BuildLaunch& L, hipStream_t stream) {
  BuildArgs a;
  a.kind = L.kind;
  a.mp = L.mp;
  a.doc_len = L.doc_len;
  a.sorted_flags = L.schedule;
  a.Bm = L.Bm;
  a.Hm = L.Hm;
  a.Q_LEN = L.Q_LEN;
  a.KV_LEN = L.KV_LEN;
  a.NQB = L.NQB;
  a.NKB = L.NKB;
  a.kv_num = L.kv_num;
  a.kv_idx = L.kv_idx;
  a.full_num = L.full_num;
  a.full_idx = L.full_idx;
  a.separate_full = L.separate_full;
  a.BS = L.block;
  a.QBS = L.q_block;
  const int rows = L.Bm * L.Hm * L.NQB;
  const size_t lds = sizeof(int) * (2 * (size_t)L.NKB + 1);
  switch (L.kind) {
    case MASK_NOOP:
      classify_kernel<MASK_NOOP><<<rows, kRowThreads, lds, stream>>>(a);
      break;
    case MASK_CAUSAL:
      classify_kernel<MASK_CAUSAL><<<rows, kRowThreads, lds, stream>>>(a);
      break;
    case MASK_SLIDING_SINK:
      classify_kernel<MASK_SLIDING_SINK><<<rows, kRowThreads, lds, stream>>>(a);
      break;
    case MASK_PREFIX_LM:
      classify_kernel<MASK_PREFIX_LM><<<rows, kRowThreads, lds, stream>>>(a);
      break;
    case MASK_COMPOSITE: {
      if (L.mp.doc) {
        const int drows = L.mp.doc_bstride > 0 ? L.Bm : 1;
        const int n = L.Q_LEN > L.KV_LEN ? L.Q_LEN : L.KV_LEN;
        const int chunk = (n + L.NQB - 1) / L.NQB;
        doc_sorted_kernel<<<dim3(L.NQB, drows), 256, 0, stream>>>(L.mp.doc, L.mp.doc_bstride, n,
                                                                 chunk, L.NQB, L.schedule);
        hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return e0;
      }
      classify_kernel<MASK_COMPOSITE><<<rows, kRowThreads, lds, stream>>>(a);
      break;
    }
    default: {
      // sortedness flags of each document row (1 or Bm rows) in NQB chunks
      const int drows = L.mp.doc_bstride > 0 ? L.Bm : 1;
      const int n = L.Q_LEN > L.KV_LEN ? L.Q_LEN : L.KV_LEN;
      const int chunk = (n + L.NQB - 1) / L.NQB;
      doc_sorted_kernel<<<dim3(L.NQB, drows), 256, 0, stream>>>(L.mp.doc, L.mp.doc_bstride, n,
                                                               chunk, L.NQB, L.schedule);
      hipError_t e0 = hipGetLastError();
      if (e0 != hipSuccess) return e0;
      classify_kernel<MASK_DOCUMENT><<<rows, kRowThreads, lds, stream>>>(a);
      break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nbins = L.NKB + 1;
  schedule_kernel<<<1, kSchedThreads, sizeof(int) * 2 * (size_t)nbins, stream>>>(
      L.kv_num, L.full_num, rows, nbins, L.schedule);
  if (L.q_num) {
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    transpose_kernel<<<L.Bm * L.Hm, kTransposeThreads, 0, stream>>>(
        L.kv_num, L.kv_idx, L.full_num, L.full_idx, L.NQB, L.NKB, L.q_num, L.q_idx,
        L.full_q_num, L.full_q_idx);
  }
  return hipGetLastError();
}

}  // namespace fa
