// Incremental updates of the HBM routing store: delete documents (compacting the
// store and its chunk offsets) and append documents, without rebuilding.
//
// chatpaper.ai page, Abstract: among the weaknesses of the alternatives it lists
// an inability to modify memory content dynamically.  Reading: deleted documents
// disappear, the survivors keep their order and are renumbered 0, 1, ...; every
// surviving document moves with all of its chunk rows (pooled router keys and,
// when the store carries them, their inverse norms); appended documents follow
// the last one.  The rows are moved, never recomputed, so an updated store is
// bit-identical to one built from scratch from the same documents.
//
//   store_scan_kernel   one workgroup: per-thread runs of documents, a workgroup
//                       scan of (kept documents, kept chunks), then each
//                       survivor's new index and new first chunk
//   store_move_kernel   one workgroup per old document: its rows, 16 bytes a lane
//   append_off_kernel   offsets of appended documents, from the device's current end
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int SCAN_THREADS = 1024;
constexpr int MOVE_THREADS = 256;

__global__ void __launch_bounds__(SCAN_THREADS)
store_scan_kernel(const int64_t* __restrict__ off, int64_t n_docs, const uint8_t* __restrict__ keep,
                  int64_t* __restrict__ off_out, int32_t* __restrict__ new_id, int64_t* __restrict__ counts) {
  __shared__ int64_t sk[SCAN_THREADS], sc[SCAN_THREADS];
  const int t = threadIdx.x;
  const int64_t per = (n_docs + SCAN_THREADS - 1) / SCAN_THREADS;
  const int64_t d0 = t * per < n_docs ? t * per : n_docs;
  const int64_t d1 = d0 + per < n_docs ? d0 + per : n_docs;
  int64_t nk = 0, nc = 0;
  for (int64_t d = d0; d < d1; ++d)
    if (keep[d]) { ++nk; nc += off[d + 1] - off[d]; }
  sk[t] = nk;
  sc[t] = nc;
  __syncthreads();
  // inclusive scan over the threads (Hillis-Steele, log2(1024) steps)
  for (int s = 1; s < SCAN_THREADS; s <<= 1) {
    const int64_t ak = t >= s ? sk[t - s] : 0, ac = t >= s ? sc[t - s] : 0;
    __syncthreads();
    sk[t] += ak;
    sc[t] += ac;
    __syncthreads();
  }
  int64_t bk = sk[t] - nk, bc = sc[t] - nc;              // exclusive bases of this thread's run
  for (int64_t d = d0; d < d1; ++d) {
    if (keep[d]) {
      new_id[d] = (int32_t)bk;
      off_out[bk] = bc;
      ++bk;
      bc += off[d + 1] - off[d];
    } else {
      new_id[d] = -1;
    }
  }
  if (t == SCAN_THREADS - 1) {
    off_out[sk[t]] = sc[t];
    counts[0] = sk[t];
    counts[1] = sc[t];
  }
}

__global__ void __launch_bounds__(MOVE_THREADS)
store_move_kernel(const uint16_t* __restrict__ rows, const float* __restrict__ norms, const int64_t* __restrict__ off,
                  const uint8_t* __restrict__ keep, const int32_t* __restrict__ new_id,
                  const int64_t* __restrict__ off_out, int row_elems, int norm_elems, uint16_t* __restrict__ rows_out,
                  float* __restrict__ norms_out) {
  const int64_t d = blockIdx.x;
  if (!keep[d]) return;
  const int64_t src = off[d], n = off[d + 1] - src;
  const int64_t dst = off_out[new_id[d]];
  // a document's rows are contiguous: n * row_elems bf16 = n * row_elems / 8 16-byte vectors
  const uint4* s = reinterpret_cast<const uint4*>(rows + src * row_elems);
  uint4* o = reinterpret_cast<uint4*>(rows_out + dst * row_elems);
  const int64_t nv = n * row_elems / 8;
  for (int64_t i = threadIdx.x; i < nv; i += MOVE_THREADS) o[i] = s[i];
  if (norms) {
    const float* sn = norms + src * norm_elems;
    float* on = norms_out + dst * norm_elems;
    for (int64_t i = threadIdx.x; i < n * norm_elems; i += MOVE_THREADS) on[i] = sn[i];
  }
}

__global__ void __launch_bounds__(256)
copy_u4_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

__global__ void __launch_bounds__(256)
append_off_kernel(int64_t* __restrict__ off, int64_t n_docs, const int64_t* __restrict__ new_off, int64_t n_new) {
  const int64_t base = off[n_docs];
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_new; i += (int64_t)gridDim.x * blockDim.x)
    off[n_docs + 1 + i] = base + new_off[i + 1];
}

}  // namespace

int launch_store_delete(const uint16_t* rows, const float* norms, const int64_t* off, int64_t n_docs, int H,
                        const uint8_t* keep, uint16_t* rows_out, float* norms_out, int64_t* off_out,
                        int32_t* new_id, int64_t* counts, hipStream_t stream) {
  hipLaunchKernelGGL(store_scan_kernel, dim3(1), dim3(SCAN_THREADS), 0, stream, off, n_docs, keep, off_out, new_id,
                     counts);
  MSA_CHECK_LAUNCH();
  hipLaunchKernelGGL(store_move_kernel, dim3((unsigned)n_docs), dim3(MOVE_THREADS), 0, stream, rows, norms, off, keep,
                     new_id, off_out, H * 128, H, rows_out, norms_out);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

int launch_store_append(uint16_t* rows, float* norms, int64_t* off, int64_t n_docs, int64_t n_chunks, int H,
                        const uint16_t* new_rows, const int64_t* new_off, int64_t n_new_docs, int64_t n_new_chunks,
                        hipStream_t stream) {
  const int64_t row_elems = (int64_t)H * 128;
  if (n_new_chunks > 0) {
    const int64_t nv = n_new_chunks * row_elems / 8;
    int64_t blocks = (nv + 255) / 256;
    blocks = blocks > 4096 ? 4096 : blocks;
    hipLaunchKernelGGL(copy_u4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(new_rows), reinterpret_cast<uint4*>(rows + n_chunks * row_elems),
                       nv);
    MSA_CHECK_LAUNCH();
    if (norms) {
      const int rc = launch_krbar_norms(rows + n_chunks * row_elems, n_new_chunks, H, norms + n_chunks * H, stream);
      if (rc != MSA_OK) return rc;
    }
  }
  if (n_new_docs > 0) {
    int64_t blocks = (n_new_docs + 255) / 256;
    blocks = blocks > 4096 ? 4096 : blocks;
    hipLaunchKernelGGL(append_off_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, off, n_docs, new_off,
                       n_new_docs);
    MSA_CHECK_LAUNCH();
  }
  return MSA_OK;
}

}  // namespace msa
