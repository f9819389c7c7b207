// Context assembly on the device (medium write-up sec. 4B and b-lab.team
// summary sec. 2: content K/V stay in host DRAM and only the selected items
// are fetched; b-lab.team pipeline stage 2: load only the selected Kbar/Vbar).
//
// One workgroup per (selected rank r, query b) copies document top_idx[b, r]'s
// chunk entries [Kbar | Vbar] from the mapped pinned host store straight into
// the staging buffer, at the offset given by the chunk counts of the ranks
// before it.  The ids never leave the GPU, so the whole route -> top-k ->
// assemble -> attend step can run without a host round trip.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int THREADS = 256;

__global__ void __launch_bounds__(THREADS)
gather_kernel(const int32_t* __restrict__ top_idx, int k, const uint16_t* __restrict__ host_store,
              const int64_t* __restrict__ doc_chunk_off, int64_t n_docs, int64_t entry_elems,
              uint16_t* __restrict__ staging, int Mmax, int32_t* __restrict__ mem_len) {
  const int r = blockIdx.x, b = blockIdx.y;
  __shared__ int64_t sh_dst, sh_src, sh_n;
  if (threadIdx.x == 0) {
    int64_t before = 0, total = 0, mine_src = 0, mine_n = 0;
    for (int q = 0; q < k; ++q) {
      const int32_t d = top_idx[(int64_t)b * k + q];
      int64_t n = 0, g0 = 0;
      if (d >= 0 && d < n_docs) {
        g0 = doc_chunk_off[d];
        n = doc_chunk_off[d + 1] - g0;
      }
      if (q < r) before += n;
      if (q == r) { mine_src = g0; mine_n = n; }
      total += n;
    }
    int64_t n = mine_n;
    if (before >= Mmax) n = 0;
    else if (before + n > Mmax) n = Mmax - before;
    sh_dst = before;
    sh_src = mine_src;
    sh_n = n;
    if (r == 0) mem_len[b] = (int32_t)(total < Mmax ? total : Mmax);
  }
  __syncthreads();
  const int64_t vecs = sh_n * entry_elems / 8;    // 16-byte vectors
  const uint4* src = reinterpret_cast<const uint4*>(host_store + sh_src * entry_elems);
  uint4* dst = reinterpret_cast<uint4*>(staging + ((int64_t)b * Mmax + sh_dst) * entry_elems);
  for (int64_t i = threadIdx.x; i < vecs; i += THREADS) dst[i] = src[i];
}

}  // namespace

int launch_gather(const int32_t* top_idx, int B, int k, const uint16_t* host_store,
                  const int64_t* doc_chunk_off, int64_t n_docs, int H, uint16_t* staging, int Mmax,
                  int32_t* mem_len, hipStream_t stream) {
  const int64_t entry_elems = 2LL * H * 128;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)k, (unsigned)B), dim3(THREADS), 0, stream, top_idx, k,
                     host_store, doc_chunk_off, n_docs, entry_elems, staging, Mmax, mem_len);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

}  // namespace msa
