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
//   store_tile_sums / store_tile_bases / store_ids   a three-pass scan of
//                       (kept documents, kept chunks) over tiles of 1,024
//                       documents: each survivor's new index and new first chunk
//   store_move_kernel   one workgroup per old document: its rows, 16 bytes a lane
//   append_off_kernel   offsets of appended documents, from the device's current end
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int TILE = 1024;          // documents per scan workgroup (one per thread)
constexpr int MOVE_THREADS = 256;
constexpr int MOVE_UNROLL = 4;      // 16-byte vectors in flight per lane

// Pass 1: per tile of TILE documents, the kept documents and their chunks.
__global__ void __launch_bounds__(TILE)
store_tile_sums_kernel(const int64_t* __restrict__ off, int64_t n_docs, const uint8_t* __restrict__ keep,
                       int64_t* __restrict__ tile_k, int64_t* __restrict__ tile_c) {
  __shared__ int64_t s_a[TILE / 64], s_b[TILE / 64];
  const int64_t d = (int64_t)blockIdx.x * TILE + threadIdx.x;
  int64_t k = 0, c = 0;
  if (d < n_docs && keep[d]) { k = 1; c = off[d + 1] - off[d]; }
  block_scan2(k, c, s_a, s_b);
  if (threadIdx.x == TILE - 1) { tile_k[blockIdx.x] = k; tile_c[blockIdx.x] = c; }
}

// Pass 2 (one workgroup): exclusive bases of the tiles, in place; totals into counts.
__global__ void __launch_bounds__(TILE)
store_tile_bases_kernel(int64_t* __restrict__ tile_k, int64_t* __restrict__ tile_c, int64_t n_tiles,
                        int64_t* __restrict__ off_out, int64_t* __restrict__ counts) {
  __shared__ int64_t s_a[TILE / 64], s_b[TILE / 64];
  __shared__ int64_t carry_k, carry_c;
  if (threadIdx.x == 0) { carry_k = 0; carry_c = 0; }
  __syncthreads();
  for (int64_t t0 = 0; t0 < n_tiles; t0 += TILE) {
    const int64_t t = t0 + threadIdx.x;
    const int64_t k0 = t < n_tiles ? tile_k[t] : 0, c0 = t < n_tiles ? tile_c[t] : 0;
    int64_t k = k0, c = c0;
    block_scan2(k, c, s_a, s_b);
    const int64_t bk = carry_k, bc = carry_c;
    if (t < n_tiles) { tile_k[t] = bk + k - k0; tile_c[t] = bc + c - c0; }
    __syncthreads();                                   // every thread has read the carry
    if (threadIdx.x == TILE - 1) { carry_k = bk + k; carry_c = bc + c; }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    off_out[carry_k] = carry_c;
    counts[0] = carry_k;
    counts[1] = carry_c;
  }
}

// Pass 3: each survivor's new index and first chunk.
__global__ void __launch_bounds__(TILE)
store_ids_kernel(const int64_t* __restrict__ off, int64_t n_docs, const uint8_t* __restrict__ keep,
                 const int64_t* __restrict__ tile_k, const int64_t* __restrict__ tile_c,
                 int64_t* __restrict__ off_out, int32_t* __restrict__ new_id) {
  __shared__ int64_t s_a[TILE / 64], s_b[TILE / 64];
  const int64_t d = (int64_t)blockIdx.x * TILE + threadIdx.x;
  const bool kept = d < n_docs && keep[d];
  const int64_t k0 = kept ? 1 : 0, c0 = kept ? off[d + 1] - off[d] : 0;
  int64_t k = k0, c = c0;
  block_scan2(k, c, s_a, s_b);
  if (d < n_docs) {
    const int64_t nk = tile_k[blockIdx.x] + k - k0;   // exclusive
    new_id[d] = kept ? (int32_t)nk : -1;
    if (kept) off_out[nk] = tile_c[blockIdx.x] + c - c0;
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
  for (int64_t i0 = threadIdx.x; i0 < nv; i0 += MOVE_THREADS * MOVE_UNROLL) {
    uint4 v[MOVE_UNROLL];
#pragma unroll
    for (int u = 0; u < MOVE_UNROLL; ++u) {
      const int64_t i = i0 + (int64_t)u * MOVE_THREADS;
      if (i < nv) v[u] = s[i];
    }
#pragma unroll
    for (int u = 0; u < MOVE_UNROLL; ++u) {
      const int64_t i = i0 + (int64_t)u * MOVE_THREADS;
      if (i < nv) o[i] = v[u];
    }
  }
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

size_t store_delete_workspace(int64_t n_docs) {
  const int64_t n_tiles = (n_docs + TILE - 1) / TILE;
  return ((size_t)2 * (size_t)n_tiles * sizeof(int64_t) + 255) & ~(size_t)255;
}

int launch_store_delete(const uint16_t* rows, const float* norms, const int64_t* off, int64_t n_docs, int H,
                        const uint8_t* keep, uint16_t* rows_out, float* norms_out, int64_t* off_out,
                        int32_t* new_id, int64_t* counts, void* workspace, hipStream_t stream) {
  const int64_t n_tiles = (n_docs + TILE - 1) / TILE;
  int64_t* tile_k = reinterpret_cast<int64_t*>(workspace);
  int64_t* tile_c = tile_k + n_tiles;
  hipLaunchKernelGGL(store_tile_sums_kernel, dim3((unsigned)n_tiles), dim3(TILE), 0, stream, off, n_docs, keep,
                     tile_k, tile_c);
  MSA_CHECK_LAUNCH();
  hipLaunchKernelGGL(store_tile_bases_kernel, dim3(1), dim3(TILE), 0, stream, tile_k, tile_c, n_tiles, off_out,
                     counts);
  MSA_CHECK_LAUNCH();
  hipLaunchKernelGGL(store_ids_kernel, dim3((unsigned)n_tiles), dim3(TILE), 0, stream, off, n_docs, keep, tile_k,
                     tile_c, off_out, new_id);
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
