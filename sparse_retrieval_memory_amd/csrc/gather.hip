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
constexpr int GATHER_SPLIT = 8;   // workgroups per selected document

__global__ void __launch_bounds__(THREADS)
gather_kernel(const int32_t* __restrict__ top_idx, int k, const uint16_t* __restrict__ host_store,
              const int64_t* __restrict__ doc_chunk_off, int64_t n_docs, int64_t entry_elems,
              uint16_t* __restrict__ staging, int Mmax, int32_t* __restrict__ mem_len) {
  const int r = blockIdx.x, b = blockIdx.y;
  __shared__ int64_t sh_dst, sh_src, sh_n;
  // where rank r's chunks go: the first wave reads the ranks' chunk counts, one lane
  // per rank (64 at a time), and prefix-sums them
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int64_t before = 0, total = 0, mine_src = 0, mine_n = 0;
    for (int q0 = 0; q0 < k; q0 += 64) {
      const int q = q0 + lane;
      int64_t n = 0, g0 = 0;
      if (q < k) {
        const int32_t d = top_idx[(int64_t)b * k + q];
        if (d >= 0 && d < n_docs) {
          g0 = doc_chunk_off[d];
          n = doc_chunk_off[d + 1] - g0;
        }
      }
      int64_t incl = n;                                  // inclusive prefix over the 64 lanes
#pragma unroll
      for (int s = 1; s < 64; s <<= 1) {
        const int64_t u = __shfl_up(incl, s);
        if (lane >= s) incl += u;
      }
      if (q == r) { mine_src = g0; mine_n = n; before = total + incl - n; }
      total += __shfl(incl, 63);
    }
    // lane r % 64 holds rank r's values; hand them to lane 0
    const int owner = r & 63;
    before = __shfl(before, owner);
    mine_src = __shfl(mine_src, owner);
    mine_n = __shfl(mine_n, owner);
    if (lane == 0) {
      int64_t n = mine_n;
      if (before >= Mmax) n = 0;
      else if (before + n > Mmax) n = Mmax - before;
      sh_dst = before;
      sh_src = mine_src;
      sh_n = n;
      if (r == 0 && blockIdx.z == 0) mem_len[b] = (int32_t)(total < Mmax ? total : Mmax);
    }
  }
  __syncthreads();
  // blockIdx.z splits one document's copy over several workgroups: reads over the host
  // link are latency-bound, so more of them in flight is what speeds the copy up
  const int64_t vecs = sh_n * entry_elems / 8;    // 16-byte vectors
  const uint4* src = reinterpret_cast<const uint4*>(host_store + sh_src * entry_elems);
  uint4* dst = reinterpret_cast<uint4*>(staging + ((int64_t)b * Mmax + sh_dst) * entry_elems);
  for (int64_t i = (int64_t)blockIdx.z * THREADS + threadIdx.x; i < vecs; i += (int64_t)gridDim.z * THREADS)
    dst[i] = src[i];
}

// Router rows for the next interleave round (medium write-up sec. 4C and
// b-lab.team summary sec. 3: documents retrieved in one round become part of
// the next round's query).  rows[b] = Qr[b] (T0 rows), then the pooled router
// keys of every chunk of ids[b, 0..n_ids) in that order, then row 0 repeated
// up to T_out rows: a repeated row leaves every token max, hence every score,
// unchanged.  One workgroup per (output row, query) copies one 2 KB row; the
// first workgroup of each query also records the row count and marks the
// listed documents as excluded (they are not selected again).
__global__ void __launch_bounds__(128)
append_rows_kernel(const uint16_t* __restrict__ Qr, int T0, const uint16_t* __restrict__ Krbar,
                   const int64_t* __restrict__ doc_chunk_off, int64_t n_docs, const int32_t* __restrict__ ids,
                   int n_ids, int T_out, int64_t row_elems, uint16_t* __restrict__ rows,
                   int32_t* __restrict__ n_rows, uint8_t* __restrict__ doc_exclude) {
  const int t = blockIdx.x, b = blockIdx.y;
  const int32_t* my_ids = ids + (int64_t)b * n_ids;
  const uint16_t* src = Qr + (int64_t)b * T0 * row_elems;            // row 0 of this query
  int64_t total = 0;
  if (t < T0) {
    src = Qr + ((int64_t)b * T0 + t) * row_elems;
  } else {
    const int64_t want = t - T0;                                        // chunk rank among the listed docs
    for (int i = 0; i < n_ids; ++i) {
      const int32_t d = my_ids[i];
      if (d < 0 || d >= n_docs) continue;
      const int64_t g0 = doc_chunk_off[d], n = doc_chunk_off[d + 1] - g0;
      if (want >= total && want < total + n) src = Krbar + (g0 + (want - total)) * row_elems;
      total += n;
    }
  }
  if (t == 0) {
    if (threadIdx.x == 0) {
      int64_t all = 0;
      for (int i = 0; i < n_ids; ++i) {
        const int32_t d = my_ids[i];
        if (d >= 0 && d < n_docs) all += doc_chunk_off[d + 1] - doc_chunk_off[d];
      }
      if (n_rows) n_rows[b] = (int32_t)(T0 + all < T_out ? T0 + all : T_out);
    }
    if (doc_exclude)
      for (int i = threadIdx.x; i < n_ids; i += blockDim.x) {
        const int32_t d = my_ids[i];
        if (d >= 0 && d < n_docs) doc_exclude[(int64_t)b * n_docs + d] = 1;
      }
  }
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(rows + ((int64_t)b * T_out + t) * row_elems);
  for (int64_t i = threadIdx.x; i < row_elems / 8; i += blockDim.x) d4[i] = s4[i];
}

}  // namespace

int launch_append_rows(const uint16_t* Qr, int B, int T0, int H, const uint16_t* Krbar,
                       const int64_t* doc_chunk_off, int64_t n_docs, const int32_t* ids, int n_ids, int T_out,
                       uint16_t* rows, int32_t* n_rows, uint8_t* doc_exclude, hipStream_t stream) {
  hipLaunchKernelGGL(append_rows_kernel, dim3((unsigned)T_out, (unsigned)B), dim3(128), 0, stream, Qr, T0, Krbar,
                     doc_chunk_off, n_docs, ids, n_ids, T_out, (int64_t)H * 128, rows, n_rows, doc_exclude);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

int launch_gather(const int32_t* top_idx, int B, int k, const uint16_t* host_store,
                  const int64_t* doc_chunk_off, int64_t n_docs, int H, uint16_t* staging, int Mmax,
                  int32_t* mem_len, hipStream_t stream) {
  const int64_t entry_elems = 2LL * H * 128;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)k, (unsigned)B, GATHER_SPLIT), dim3(THREADS), 0, stream, top_idx, k,
                     host_store, doc_chunk_off, n_docs, entry_elems, staging, Mmax, mem_len);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

}  // namespace msa
