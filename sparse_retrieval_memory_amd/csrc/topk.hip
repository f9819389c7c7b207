// Top-k document selection (medium write-up sec. 2; b-lab.team summary sec. 1
// and pipeline stage 2; jkf87 blog, core technique 1: keep the k most relevant
// documents).
//
// Each document becomes one 64-bit key (order-preserving score bits << 32 |
// ~doc_id), so "score descending, ties to the lower id" is plain descending
// integer order and every key is unique -- the selection is exact and
// deterministic.  Two passes of the same block-level routine:
//   pass 1: (blocks x B) workgroups each reduce a slice of documents to its k
//           best keys;
//   pass 2: one workgroup per query reduces the blocks' candidates to k.
// The block routine keeps a running top-k in LDS and repeatedly bitonic-sorts
// it together with the next SORT_N - k keys.
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

int64_t pass1_blocks(int64_t n_docs, int k) {
  const int64_t piece = SORT_N - k;
  return (n_docs + piece - 1) / piece;
}

}  // namespace

size_t topk_workspace(int B, int64_t n_docs, int k) {
  if (k < 1 || k > KMAX) return 0;
  return (size_t)B * (size_t)pass1_blocks(n_docs, k) * (size_t)k * sizeof(uint64_t);
}

int launch_topk(const float* doc_scores, int B, int64_t n_docs, int k, int32_t* top_idx,
                float* top_scores, void* workspace, hipStream_t stream) {
  if (k > KMAX) {
    set_error("k=%d exceeds the supported maximum %d", k, KMAX);
    return MSA_ERR_UNSUPPORTED;
  }
  const int64_t nb = pass1_blocks(n_docs, k);
  const int64_t slice = SORT_N - k;
  uint64_t* cand = reinterpret_cast<uint64_t*>(workspace);
  hipLaunchKernelGGL(topk_pass1, dim3((unsigned)nb, (unsigned)B), dim3(THREADS), 0, stream, doc_scores,
                     n_docs, k, slice, cand);
  MSA_CHECK_LAUNCH();
  hipLaunchKernelGGL(topk_pass2, dim3((unsigned)B), dim3(THREADS), 0, stream, cand, nb * (int64_t)k, k,
                     top_idx, top_scores);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

}  // namespace msa
