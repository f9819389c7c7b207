// Top-k document selection (medium write-up sec. 2; b-lab.team summary sec. 1
// and pipeline stage 2; jkf87 blog, core technique 1: keep the k most relevant
// documents).
//
// Each document becomes one 64-bit key (order-preserving score bits << 32 |
// ~doc_id), so "score descending, ties to the lower id" is plain descending
// integer order and every key is unique -- the selection is exact and
// deterministic.  k <= 32 (the workloads use 4, 8 and 16): group maxima, then
// only the winning groups are searched (below).  Larger k: two passes of a
// block-level routine -- pass 1: (blocks x B) workgroups each reduce a slice
// of documents to its k best keys; pass 2: one workgroup per query reduces the
// blocks' candidates to k -- which keeps a running top-k in LDS and
// repeatedly bitonic-sorts it together with the next SORT_N - k keys.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int SORT_N = 2048;
constexpr int THREADS = 256;
constexpr int KMAX = 1024;

__device__ __forceinline__ uint64_t make_key(float s, uint32_t id) {
  return ((uint64_t)enc_f32(s) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

__device__ void bitonic_sort_desc(uint64_t* s) {
  for (int size = 2; size <= SORT_N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < SORT_N / 2; i += THREADS) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t a = s[lo], b = s[hi];
        if ((a < b) == desc) { s[lo] = b; s[hi] = a; }
      }
      __syncthreads();
    }
  }
}

// Reduce keys get(0..count-1) to the k largest, left in s[0..k) (descending).
template <typename Get>
__device__ void block_topk(uint64_t* s, int64_t count, int k, Get get) {
  for (int i = threadIdx.x; i < k; i += THREADS) s[i] = 0;
  const int piece = SORT_N - k;
  for (int64_t base = 0; base < count || base == 0; base += piece) {
    for (int i = threadIdx.x; i < piece; i += THREADS) {
      const int64_t x = base + i;
      s[k + i] = x < count ? get(x) : 0ull;
    }
    __syncthreads();
    bitonic_sort_desc(s);
    if (base + piece >= count) break;
  }
}

__global__ void __launch_bounds__(THREADS)
topk_pass1(const float* __restrict__ scores, int64_t n_docs, int k, int64_t slice,
           uint64_t* __restrict__ cand) {
  __shared__ uint64_t s[SORT_N];
  const int b = blockIdx.y;
  const int64_t d0 = (int64_t)blockIdx.x * slice;
  int64_t cnt = n_docs - d0;
  if (cnt > slice) cnt = slice;
  if (cnt < 0) cnt = 0;
  const float* row = scores + (int64_t)b * n_docs;
  block_topk(s, cnt, k, [&](int64_t x) { return make_key(row[d0 + x], (uint32_t)(d0 + x)); });
  uint64_t* out = cand + ((int64_t)b * gridDim.x + blockIdx.x) * k;
  for (int i = threadIdx.x; i < k; i += THREADS) out[i] = s[i];
}

__global__ void __launch_bounds__(THREADS)
topk_pass2(const uint64_t* __restrict__ cand, int64_t n_cand, int k, int32_t* __restrict__ top_idx,
           float* __restrict__ top_scores) {
  __shared__ uint64_t s[SORT_N];
  const int b = blockIdx.x;
  const uint64_t* row = cand + (int64_t)b * n_cand;
  block_topk(s, n_cand, k, [&](int64_t x) { return row[x]; });
  for (int i = threadIdx.x; i < k; i += THREADS) {
    const uint64_t key = s[i];
    top_idx[(int64_t)b * k + i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
    top_scores[(int64_t)b * k + i] = dec_f32((uint32_t)(key >> 32));
  }
}

// ---------------------------------------------------------------- small k
// k <= 32.  Group the documents in runs of 64 (one wave) and take each group's
// best key.  Every one of the k best documents sits in a group whose best key
// is at least its own, and distinct such groups have distinct best keys, so
// the k best documents lie inside the k groups with the largest best keys.
//   pass 1 (many workgroups): group maxima by a wave-wide max of 64-bit keys;
//   pass 2 (one workgroup per query): each wave extracts the top k of its
//           share of the group maxima from registers, one wave merges the
//           lists, then the k winning groups' 64 documents each are gathered
//           and reduced the same way.  Extraction needs no barriers or LDS
//           sorts, which is what makes it fast at these sizes.
constexpr int GROUP = 64;

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

__global__ void __launch_bounds__(256)
topk_group_max(const float* __restrict__ scores, int64_t n_docs, int64_t n_groups, uint64_t* __restrict__ gmax) {
  const int b = blockIdx.y;
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint64_t key = d < n_docs ? make_key(scores[(int64_t)b * n_docs + d], (uint32_t)d) : 0ull;
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    const uint64_t o = shfl_xor_u64(key, m);
    key = o > key ? o : key;
  }
  const int64_t g = d / GROUP;
  if ((threadIdx.x & 63) == 0 && g < n_groups) gmax[(int64_t)b * n_groups + g] = key;
}

// Max over the wave of a 32-bit value, returned uniformly: prefix max inside
// each row of 16 (row_shr 1, 2, 4, 8), then rows 1 and 3 take lane 15 of the
// row below (row_bcast 15) and rows 2 and 3 take lane 31 (row_bcast 31), so
// lane 63 holds the total.  Lanes without a source read 0, the identity.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true); v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true); v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true); v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true); v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, true); v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, true); v = o > v ? o : v;
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Largest 64-bit key of the wave: the high words (the score) decide unless
// several lanes share the largest one, then the low words (the id) do.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
  const uint32_t mh = wave_max_u32(hi);
  const uint64_t tie = __ballot(hi == mh);
  uint32_t ml;
  if (__popcll(tie) == 1)
    ml = (uint32_t)__builtin_amdgcn_readlane((int)lo, __ffsll((unsigned long long)tie) - 1);
  else
    ml = wave_max_u32(hi == mh ? lo : 0u);
  return ((uint64_t)mh << 32) | ml;
}

// Wave-wide top-k by extraction: every lane holds R keys in registers (0 =
// empty); k rounds of a wave argmax, the winning lane drops its key.  Lane r
// ends with the r-th largest key (r < k).  No barriers, no LDS.
template <int R>
__device__ __forceinline__ uint64_t wave_extract_topk(uint64_t (&kv)[R], int k, int lane) {
  uint64_t lm = 0;
#pragma unroll
  for (int j = 0; j < R; ++j) lm = kv[j] > lm ? kv[j] : lm;
  uint64_t mine = 0;
  for (int r = 0; r < k; ++r) {
    const uint64_t m = wave_max_key(lm);
    if (lane == r) mine = m;
    if (m != 0ull && lm == m) {               // keys are unique: exactly one lane owns m
      lm = 0;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        kv[j] = kv[j] == m ? 0ull : kv[j];
        lm = kv[j] > lm ? kv[j] : lm;
      }
    }
  }
  return mine;
}

constexpr int P2_WAVES = 16;
constexpr int RA = 5;                         // group keys per lane per sweep (4 new + the running list)

// Top k of P2_WAVES lists of k keys each (lists[w][r], r < k) by one wave;
// key x = w * k + r sits in lane x % 64, slot x / 64 (RM = ceil(16 k / 64)).
template <int RM>
__device__ __forceinline__ uint64_t merge_lists(const uint64_t (*lists)[64], int k, int lane) {
  uint64_t kv[RM];
#pragma unroll
  for (int j = 0; j < RM; ++j) {
    const int x = j * 64 + lane;
    kv[j] = x < P2_WAVES * k ? lists[x / k][x % k] : 0ull;
  }
  return wave_extract_topk<RM>(kv, k, lane);
}

// Phase A of the general path: each wave keeps a running top k over its share
// of `n` keys (key(x), x < n), then one wave merges the lists; lane r of the
// result holds the r-th largest key (0 past the end).  All threads must call it.
template <int RM, typename Get>
__device__ __forceinline__ void topk_by_waves(int64_t n, int k, Get key, uint64_t (*lists)[64], uint64_t* out,
                                              int wave, int lane) {
  const int64_t per = (n + P2_WAVES - 1) / P2_WAVES;
  const int64_t g0 = wave * per;
  const int64_t g1 = (g0 + per < n) ? g0 + per : n;
  uint64_t run = 0;                           // lane r < k: the wave's r-th best so far
  for (int64_t base = g0;; base += 64 * (RA - 1)) {
    uint64_t kv[RA];
#pragma unroll
    for (int j = 0; j < RA - 1; ++j) {
      const int64_t x = base + (int64_t)j * 64 + lane;
      kv[j] = x < g1 ? key(x) : 0ull;
    }
    kv[RA - 1] = run;
    run = wave_extract_topk<RA>(kv, k, lane);
    if (base + 64 * (RA - 1) >= g1) break;
  }
  lists[wave][lane] = run;
  __syncthreads();
  if (wave == 0) out[lane] = merge_lists<RM>(lists, k, lane);
  __syncthreads();
}

// Set a query's group maxima back to 0 once every wave is past its last read of them
// (the routing workspace is handed back cleared; see launch_docs_topk).
__device__ __forceinline__ void clear_groups(uint64_t* gm, int64_t n_groups) {
  __syncthreads();
  for (int64_t x = threadIdx.x; x < n_groups; x += blockDim.x) gm[x] = 0ull;
}

template <int RM, int RB>   // RM: merge keys per lane; RB = ceil(k / P2_WAVES) winning groups per wave
__global__ void __launch_bounds__(64 * P2_WAVES)
topk_from_groups(const float* __restrict__ scores, uint64_t* __restrict__ gmax, int64_t n_docs,
                 int64_t n_groups, int k, int32_t* __restrict__ top_idx, float* __restrict__ top_scores,
                 int clear) {
  __shared__ uint64_t lists[P2_WAVES][64];
  __shared__ uint64_t groups[64];
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t* gm = gmax + (int64_t)b * n_groups;

  // A: the k best group maxima
  topk_by_waves<RM>(n_groups, k, [&](int64_t x) { return gm[x]; }, lists, groups, wave, lane);

  // B: the k winning groups' documents; wave w takes groups w, w + P2_WAVES, ...
  const float* row = scores + (int64_t)b * n_docs;
  uint64_t kv[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int r = wave + j * P2_WAVES;
    uint64_t key = 0;
    if (r < k && groups[r] != 0ull) {
      const uint32_t best_doc = 0xFFFFFFFFu - (uint32_t)(groups[r] & 0xFFFFFFFFull);
      const int64_t d = (int64_t)(best_doc / GROUP) * GROUP + lane;
      if (d < n_docs) key = make_key(row[d], (uint32_t)d);
    }
    kv[j] = key;
  }
  const uint64_t best = wave_extract_topk<RB>(kv, k, lane);
  __syncthreads();                            // everyone has read `groups` and the lists
  lists[wave][lane] = best;
  __syncthreads();
  if (wave == 0) {
    const uint64_t key = merge_lists<RM>(lists, k, lane);
    if (lane < k) {
      top_idx[(int64_t)b * k + lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
      top_scores[(int64_t)b * k + lane] = dec_f32((uint32_t)(key >> 32));
    }
  }
  if (clear) clear_groups(gmax + (int64_t)b * n_groups, n_groups);
}

// k <= P2_WAVES: the same two selections, each preceded by a threshold that
// drops almost every key before any extraction.
//   A: every wave takes the maximum of its share of the group maxima; these
//      are P2_WAVES distinct keys, so the k-th largest of them (T0) is at most
//      the k-th largest group maximum, and the k winning groups all have keys
//      >= T0.  Keys >= T0 are appended to an LDS list.
//   B: the k winning groups' best documents are k distinct documents with keys
//      >= T1 = the k-th winning group's key, so the k best documents all have
//      keys >= T1; those are appended to the list.
// A list of at most 256 keys is ranked in one step (reduce_list); a longer one
// is reduced by all waves and a merge; if phase A's list would overflow LDS
// (adversarial score layouts), the unfiltered path runs instead.
constexpr int LIST_CAP = 1024;
constexpr int GPL = 4;                        // group maxima per lane loaded in one batch

// A list of n <= RANK_MAX keys is reduced by ranking: 4 threads per key count the
// keys above it (keys are unique, so the ranks are 0..n-1), and the key of rank r < k
// goes to out[r]; out[n..63] are cleared.  Longer lists: waves + merge.
constexpr int RANK_MAX = 16 * P2_WAVES;

template <int RM>
__device__ __forceinline__ void reduce_list(const uint64_t* list, int n, int k, uint64_t (*lists)[64], uint64_t* out,
                                            int wave, int lane) {
  if (n <= RANK_MAX) {                        // uniform branch: n is read from LDS after a barrier
    const int t = threadIdx.x, i = t >> 2, part = t & 3;
    const uint64_t key = i < n ? list[i] : 0ull;
    int above = 0;
    for (int j = part; j < n; j += 4) above += list[j] > key;
    above += __shfl_xor(above, 1);
    above += __shfl_xor(above, 2);
    if (i < n && part == 0 && above < k) out[above] = key;
    if (t >= n && t < 64) out[t] = 0ull;
    __syncthreads();
  } else {
    topk_by_waves<RM>(n, k, [&](int64_t x) { return list[x]; }, lists, out, wave, lane);
  }
}

// Append the keys of `kv` that are >= t (and not empty) to list[*count ...].
__device__ __forceinline__ void append_ge(uint64_t key, uint64_t t, uint64_t* list, int* count, int lane) {
  const bool keep = key != 0ull && key >= t;
  const uint64_t mask = __ballot(keep);
  if (mask == 0ull) return;
  int base = 0;
  if (lane == 0) base = atomicAdd(count, __popcll(mask));
  base = __shfl(base, 0);
  const int pos = base + __popcll(mask & ((1ull << lane) - 1ull));
  if (keep && pos < LIST_CAP) list[pos] = key;
}

template <int RM>
__global__ void __launch_bounds__(64 * P2_WAVES)
topk_from_groups_filtered(const float* __restrict__ scores, uint64_t* __restrict__ gmax, int64_t n_docs,
                          int64_t n_groups, int k, int32_t* __restrict__ top_idx, float* __restrict__ top_scores,
                          int clear) {
  __shared__ uint64_t lists[P2_WAVES][64];
  __shared__ uint64_t groups[64];
  __shared__ uint64_t list[LIST_CAP];
  __shared__ uint64_t wmax[P2_WAVES];
  __shared__ uint64_t thresh;
  __shared__ int count;
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t* gm = gmax + (int64_t)b * n_groups;
  const int64_t per = (n_groups + P2_WAVES - 1) / P2_WAVES;
  const int64_t g0 = wave * per;
  const int64_t g1 = (g0 + per < n_groups) ? g0 + per : n_groups;

  // A1: wave maxima, then T0 = the k-th largest of them (0 if fewer than k are non-empty).
  // Up to 64 * GPL group maxima per wave stay in registers for A2; the loads of a batch are
  // issued together so their latencies overlap.
  const bool in_regs = per <= 64 * GPL;
  uint64_t gv[GPL];
  uint64_t lm = 0;
  for (int64_t base = g0; base < g1; base += 64 * GPL) {
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const int64_t x = base + j * 64 + lane;
      gv[j] = x < g1 ? gm[x] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < GPL; ++j) lm = gv[j] > lm ? gv[j] : lm;
  }
  const uint64_t wm = wave_max_key(lm);
  if (lane == 0) wmax[wave] = wm;
  if (threadIdx.x == 0) { thresh = 0; count = 0; }
  __syncthreads();
  if (threadIdx.x < P2_WAVES) {
    const uint64_t mine = wmax[threadIdx.x];
    int rank = 0;
#pragma unroll
    for (int j = 0; j < P2_WAVES; ++j) rank += wmax[j] > mine;
    if (rank == k - 1 && mine != 0ull) thresh = mine;   // keys are unique, so one lane at most
  }
  __syncthreads();
  // A2: keys >= T0 into the list
  const uint64_t t0 = thresh;
  if (in_regs) {
#pragma unroll
    for (int j = 0; j < GPL; ++j)
      if (g0 + j * 64 < g1) append_ge(gv[j], t0, list, &count, lane);
  } else {
    for (int64_t base = g0; base < g1; base += 64 * GPL) {
#pragma unroll
      for (int j = 0; j < GPL; ++j) {
        const int64_t x = base + j * 64 + lane;
        gv[j] = x < g1 ? gm[x] : 0ull;
      }
#pragma unroll
      for (int j = 0; j < GPL; ++j) append_ge(gv[j], t0, list, &count, lane);
    }
  }
  __syncthreads();
  const int na = count;
  if (na > LIST_CAP) {
    topk_by_waves<RM>(n_groups, k, [&](int64_t x) { return gm[x]; }, lists, groups, wave, lane);
  } else {
    reduce_list<RM>(list, na, k, lists, groups, wave, lane);
  }

  // B: documents of the k winning groups that are >= T1 (wave w takes group w)
  const uint64_t t1 = groups[k - 1];
  __syncthreads();                            // every wave has read `groups[k - 1]` and na
  if (threadIdx.x == 0) count = 0;
  __syncthreads();
  const float* row = scores + (int64_t)b * n_docs;
  if (wave < k && groups[wave] != 0ull) {
    const uint32_t best_doc = 0xFFFFFFFFu - (uint32_t)(groups[wave] & 0xFFFFFFFFull);
    const int64_t d = (int64_t)(best_doc / GROUP) * GROUP + lane;
    append_ge(d < n_docs ? make_key(row[d], (uint32_t)d) : 0ull, t1, list, &count, lane);
  }
  __syncthreads();
  const int nb = count;                       // <= k * 64 <= LIST_CAP
  reduce_list<RM>(list, nb, k, lists, groups, wave, lane);
  if (wave == 0 && lane < k) {
    const uint64_t key = groups[lane];
    top_idx[(int64_t)b * k + lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
    top_scores[(int64_t)b * k + lane] = dec_f32((uint32_t)(key >> 32));
  }
  if (clear) clear_groups(gm, n_groups);
}

// The document max (the last step of the routing scores: a document's score is the max of its
// chunks', -inf when excluded or empty), with the group maxima of the top-k folded in (GROUPS).
// One workgroup of 128 threads per (group of 64 documents, query), so that every workgroup of a
// 100M-token layer's 3,125 groups is resident at once and the kernel costs about one workgroup's
// latency.  Offsets are non-decreasing, so the group's documents own the contiguous chunk range
// [off[d0], off[d0 + nd]): the threads read it and set it back to 0 (re-arming the workspace for
// the next scan) with coalesced accesses, DR_BATCH chunks in flight per thread (one pass for up to
// 1,024 chunks), and each chunk finds its document by a binary search over the group's offsets in
// LDS and adds its maximum to the document's LDS slot with an LDS atomic max; then the first wave
// forms the 64 scores and the group's largest key.  The exclusion flags are loaded with the
// offsets, before the first barrier.  Offsets are clamped to [0, n_chunks] and the search stays
// inside the group, so offsets that break the contract give wrong scores but no access outside
// the buffers.
constexpr int DR_THREADS = 128;
constexpr int DR_BATCH = 8;

template <bool GROUPS>
__global__ void __launch_bounds__(DR_THREADS)
doc_reduce_kernel(uint32_t* __restrict__ chunk_enc, int64_t n_chunks,
                  const int64_t* __restrict__ doc_chunk_off, int64_t n_docs,
                  const uint8_t* __restrict__ doc_exclude, float* __restrict__ doc_scores,
                  float* __restrict__ chunk_scores, int64_t n_groups, uint64_t* __restrict__ gmax) {
  __shared__ int64_t s_off[GROUP + 1];
  __shared__ uint32_t s_best[GROUP];
  const int b = blockIdx.y;
  const int64_t grp = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t d0 = grp * GROUP;
  const int nd = (int)(n_docs - d0 < GROUP ? n_docs - d0 : GROUP);   // >= 1
  bool excluded = false;
  if (doc_exclude && tid < nd) excluded = doc_exclude[(int64_t)b * n_docs + d0 + tid] != 0;
  if (tid <= nd) {
    int64_t o = doc_chunk_off[d0 + tid];
    o = o < 0 ? 0 : (o > n_chunks ? n_chunks : o);
    s_off[tid] = o;
  }
  if (tid < GROUP) s_best[tid] = 0u;
  __syncthreads();
  const int64_t c0 = s_off[0], c1 = s_off[nd];
  uint32_t* ce = chunk_enc + (int64_t)b * n_chunks;
  float* cs = chunk_scores ? chunk_scores + (int64_t)b * n_chunks : nullptr;
  // the largest j < nd with s_off[j] <= c (for c0 <= c < c1: the non-empty document holding c)
  auto doc_of = [&](int64_t c) {
    int lo = 0, hi = nd;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_off[mid] <= c) lo = mid;
      else hi = mid;
    }
    return lo;
  };
  for (int64_t c = c0 + tid; c < c1; c += DR_THREADS * DR_BATCH) {
    uint32_t e[DR_BATCH];
#pragma unroll
    for (int u = 0; u < DR_BATCH; ++u) {
      const int64_t cu = c + u * DR_THREADS;
      e[u] = cu < c1 ? ce[cu] : 0u;
    }
#pragma unroll
    for (int u = 0; u < DR_BATCH; ++u) {
      const int64_t cu = c + u * DR_THREADS;
      if (cu < c1) {
        ce[cu] = 0u;
        if (cs) cs[cu] = dec_f32(e[u]);
        atomicMax(&s_best[doc_of(cu)], e[u]);
      }
    }
  }
  __syncthreads();
  if (tid < GROUP) {
    uint64_t key = 0ull;
    if (tid < nd) {
      const int64_t d = d0 + tid;
      float s = s_off[tid + 1] > s_off[tid] ? dec_f32(s_best[tid]) : -INFINITY;
      if (excluded) s = -INFINITY;
      doc_scores[(int64_t)b * n_docs + d] = s;
      key = make_key(s, (uint32_t)d);
    }
    if constexpr (GROUPS) {
#pragma unroll
      for (int m = 32; m > 0; m >>= 1) {
        const uint64_t o = shfl_xor_u64(key, m);
        key = o > key ? o : key;
      }
      if (tid == 0) gmax[(int64_t)b * n_groups + grp] = key;
    }
  }
}

// The group-based selection from group maxima already in gmax (1 <= k <= 32).
int launch_topk_from_groups(const float* doc_scores, int B, int64_t n_docs, int k, int32_t* top_idx,
                            float* top_scores, uint64_t* gmax, int clear, hipStream_t stream) {
  const int64_t n_groups = (n_docs + GROUP - 1) / GROUP;
#define MSA_TOPK_GROUPS(RMV, RBV)                                                                        \
  hipLaunchKernelGGL((topk_from_groups<RMV, RBV>), dim3((unsigned)B), dim3(64 * P2_WAVES), 0, stream, doc_scores, \
                     gmax, n_docs, n_groups, k, top_idx, top_scores, clear)
#define MSA_TOPK_FILTERED(RMV)                                                                          \
  hipLaunchKernelGGL((topk_from_groups_filtered<RMV>), dim3((unsigned)B), dim3(64 * P2_WAVES), 0, stream,     \
                     doc_scores, gmax, n_docs, n_groups, k, top_idx, top_scores, clear)
  if (k <= 4) MSA_TOPK_FILTERED(1);
  else if (k <= 8) MSA_TOPK_FILTERED(2);
  else if (k <= 16) MSA_TOPK_FILTERED(4);
  else MSA_TOPK_GROUPS(8, 2);
#undef MSA_TOPK_GROUPS
#undef MSA_TOPK_FILTERED
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

int launch_topk_small(const float* doc_scores, int B, int64_t n_docs, int k, int32_t* top_idx, float* top_scores,
                      uint64_t* gmax, hipStream_t stream) {
  const int64_t n_groups = (n_docs + GROUP - 1) / GROUP;
  hipLaunchKernelGGL(topk_group_max, dim3((unsigned)((n_docs + 255) / 256), (unsigned)B), dim3(256), 0, stream,
                     doc_scores, n_docs, n_groups, gmax);
  MSA_CHECK_LAUNCH();
  return launch_topk_from_groups(doc_scores, B, n_docs, k, top_idx, top_scores, gmax, 0, stream);
}

int64_t pass1_blocks(int64_t n_docs, int k) {
  const int64_t piece = SORT_N - k;
  return (n_docs + piece - 1) / piece;
}

}  // namespace

int launch_docs_topk(uint32_t* chunk_enc, int64_t n_chunks, const int64_t* doc_chunk_off, int64_t n_docs,
                     const uint8_t* doc_exclude, int B, int k, float* doc_scores, float* chunk_scores,
                     int32_t* top_idx, float* top_scores, uint64_t* gmax, hipStream_t stream) {
  const int64_t n_groups = (n_docs + GROUP - 1) / GROUP;
  hipLaunchKernelGGL(doc_reduce_kernel<true>, dim3((unsigned)n_groups, (unsigned)B), dim3(DR_THREADS), 0, stream,
                     chunk_enc, n_chunks, doc_chunk_off, n_docs, doc_exclude, doc_scores, chunk_scores, n_groups,
                     gmax);
  MSA_CHECK_LAUNCH();
  return launch_topk_from_groups(doc_scores, B, n_docs, k, top_idx, top_scores, gmax, 1, stream);
}

int launch_doc_reduce(uint32_t* chunk_enc, int64_t n_chunks, const int64_t* doc_chunk_off, int64_t n_docs,
                      const uint8_t* doc_exclude, int B, float* doc_scores, float* chunk_scores, hipStream_t stream) {
  const int64_t n_groups = (n_docs + GROUP - 1) / GROUP;
  hipLaunchKernelGGL(doc_reduce_kernel<false>, dim3((unsigned)n_groups, (unsigned)B), dim3(DR_THREADS), 0, stream,
                     chunk_enc, n_chunks, doc_chunk_off, n_docs, doc_exclude, doc_scores, chunk_scores, n_groups,
                     nullptr);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

size_t topk_workspace(int B, int64_t n_docs, int k) {
  if (k < 1 || k > KMAX) return 0;
  if (k <= 32) return (size_t)B * (size_t)((n_docs + GROUP - 1) / GROUP) * sizeof(uint64_t);
  return (size_t)B * (size_t)pass1_blocks(n_docs, k) * (size_t)k * sizeof(uint64_t);
}

int launch_topk(const float* doc_scores, int B, int64_t n_docs, int k, int32_t* top_idx,
                float* top_scores, void* workspace, hipStream_t stream) {
  if (k > KMAX) {
    set_error("k=%d exceeds the supported maximum %d", k, KMAX);
    return MSA_ERR_UNSUPPORTED;
  }
  uint64_t* cand = reinterpret_cast<uint64_t*>(workspace);
  if (k <= 32) return launch_topk_small(doc_scores, B, n_docs, k, top_idx, top_scores, cand, stream);
  const int64_t nb = pass1_blocks(n_docs, k);
  const int64_t slice = SORT_N - k;
  hipLaunchKernelGGL(topk_pass1, dim3((unsigned)nb, (unsigned)B), dim3(THREADS), 0, stream, doc_scores,
                     n_docs, k, slice, cand);
  MSA_CHECK_LAUNCH();
  hipLaunchKernelGGL(topk_pass2, dim3((unsigned)B), dim3(THREADS), 0, stream, cand, nb * (int64_t)k, k,
                     top_idx, top_scores);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

}  // namespace msa
