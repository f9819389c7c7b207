// Router-key encoding: project every token's hidden state and chunk-mean pool it
// (offline Global Memory Encoding of K_r).
//
// b-lab.team summary, pipeline stage "Global Memory Encoding": a forward pass
// over the corpus caches the chunk-pooled (K, V, K_r); sec. 1: the router key
// of a document is pooled per chunk like K and V, and a router projector maps
// hidden states to the routing space.  Reading: K_r,t = h_t W^T (W stored
// [H*D, d_model], no bias), Krbar[g] = mean over chunk g's tokens of K_r,t.
//
// The projection is linear, so the chunk mean of the projections equals the
// projection of the chunk's mean hidden state; the kernels use that order,
// which moves d_model / (H*D) times fewer bytes through the matrix cores and
// leaves the stream of hidden states as the only large cost:
//   1. hidden_pool_kernel (HBM-bound): one workgroup per chunk sums its tokens'
//      hidden rows in fp32 and writes the mean as a bf16 hi + lo pair
//      (hi = RNE(mean), lo = RNE(mean - hi): ~2^-17 relative), [n_chunks, d_model]
//      each, into the workspace;
//   2. proj_gemm_kernel (matrix cores): Krbar^T = W (hi + lo)^T with
//      v_mfma_f32_32x32x16_bf16 (exact bf16 products, fp32 accumulation), tiles
//      of 128 features x 128 chunks staged through LDS, then rounded to bf16.
#include "msa_internal.h"

namespace msa {
namespace {

// ------------------------------------------------------------ 1. pooling
constexpr int POOL_UNROLL = 8;   // token rows in flight per lane

// Document of chunk g (doc_chunk_off[d] <= g < doc_chunk_off[d+1]) by a 64-way
// search: every lane of the calling wave tests one pivot per step.
__device__ __forceinline__ int64_t find_doc64(const int64_t* __restrict__ doc_chunk_off, int64_t n_docs, int64_t g,
                                              int lane) {
  int64_t lo = 0, hi = n_docs;
  while (hi - lo > 1) {
    const int64_t span = hi - lo;
    const int64_t piv = lo + (span * lane) / 64;
    const uint64_t mask = __ballot(doc_chunk_off[piv] <= g);
    const int c = __popcll(mask);                      // pivots at or below g form a prefix
    const int64_t nlo = lo + (span * (c - 1)) / 64;
    const int64_t nhi = (c < 64) ? lo + (span * c) / 64 : hi;
    lo = nlo;
    hi = nhi > nlo ? nhi : nlo + 1;
  }
  return lo;
}

// blockDim.x >= d_model / 8: lane v owns dims [8v, 8v + 8) of the chunk's mean.
__global__ void __launch_bounds__(1024)
hidden_pool_kernel(const uint16_t* __restrict__ hidden, int64_t n_tok, int dm,
                   const int64_t* __restrict__ doc_tok_off, const int64_t* __restrict__ doc_chunk_off,
                   int64_t n_docs, int chunk_len, uint16_t* __restrict__ mean_hi,
                   uint16_t* __restrict__ mean_lo) {
  __shared__ int64_t sh_doc;
  const int tid = threadIdx.x;
  const int64_t gl = blockIdx.x;                       // output row
  const int64_t g = doc_chunk_off[0] + gl;             // global chunk index
  if (tid < 64) {
    const int64_t d = find_doc64(doc_chunk_off, n_docs, g, tid);
    if (tid == 0) sh_doc = d;
  }
  __syncthreads();
  const int64_t d = sh_doc;
  const int64_t j = g - doc_chunk_off[d];
  const int64_t L = doc_tok_off[d + 1] - doc_tok_off[d];
  const int64_t p0 = j * chunk_len;
  int cnt = (int)((L - p0) < chunk_len ? (L - p0) : chunk_len);
  const int64_t row0 = doc_tok_off[d] - doc_tok_off[0] + p0;
  if (cnt < 0 || row0 < 0 || row0 + cnt > n_tok) cnt = 0;   // inconsistent offsets: write zeros

  const int nv = dm / 8;
  if (tid >= nv) return;
  const uint16_t* src = hidden + row0 * dm + 8 * tid;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  int t = 0;
  for (; t + POOL_UNROLL <= cnt; t += POOL_UNROLL) {
    uint4 v[POOL_UNROLL];
#pragma unroll
    for (int u = 0; u < POOL_UNROLL; ++u) v[u] = load_nt16(src + (int64_t)(t + u) * dm);
#pragma unroll
    for (int u = 0; u < POOL_UNROLL; ++u) {
      acc[0] += bf16_lo(v[u].x); acc[1] += bf16_hi(v[u].x);
      acc[2] += bf16_lo(v[u].y); acc[3] += bf16_hi(v[u].y);
      acc[4] += bf16_lo(v[u].z); acc[5] += bf16_hi(v[u].z);
      acc[6] += bf16_lo(v[u].w); acc[7] += bf16_hi(v[u].w);
    }
  }
  for (; t < cnt; ++t) {
    const uint4 v = load_nt16(src + (int64_t)t * dm);
    acc[0] += bf16_lo(v.x); acc[1] += bf16_hi(v.x);
    acc[2] += bf16_lo(v.y); acc[3] += bf16_hi(v.y);
    acc[4] += bf16_lo(v.z); acc[5] += bf16_hi(v.z);
    acc[6] += bf16_lo(v.w); acc[7] += bf16_hi(v.w);
  }
  const float inv = cnt > 0 ? 1.0f / (float)cnt : 0.f;
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = acc[2 * e] * inv, b = acc[2 * e + 1] * inv;
    const uint32_t ha = f32_to_bf16_rne(a), hb = f32_to_bf16_rne(b);
    h[e] = ha | (hb << 16);
    l[e] = f32_to_bf16_rne(a - __uint_as_float(ha << 16)) | (f32_to_bf16_rne(b - __uint_as_float(hb << 16)) << 16);
  }
  *reinterpret_cast<uint4*>(mean_hi + gl * dm + 8 * tid) = make_uint4(h[0], h[1], h[2], h[3]);
  *reinterpret_cast<uint4*>(mean_lo + gl * dm + 8 * tid) = make_uint4(l[0], l[1], l[2], l[3]);
}

// ------------------------------------------------------- 2. projection GEMM
constexpr int GT = 128;              // features (n) and chunks (m) per workgroup tile
constexpr int KS = 32;               // k per LDS stage (2 MFMA k-steps)
constexpr int GTHREADS = 256;        // 4 waves, each 64 features x 64 chunks
constexpr int ROWB = KS * 2 + 16;    // LDS bytes per staged row: 64 B + 16 B skew (conflict-free reads)
constexpr int TILEB = GT * ROWB;     // one operand tile in LDS

// Krbar[m, n] = sum_k W[n, k] * (P_hi[m, k] + P_lo[m, k]) for n < N (= H*D), m < M.
// MFMA orientation: A = W rows (lane: feature l%32, k 8(l/32)+j), B = P rows
// (lane: chunk l%32, same k), so a lane's result holds 4 consecutive features
// of one chunk per 4 accumulators -- one 8-byte store into the chunk's row.
__global__ void __launch_bounds__(GTHREADS, 2)
proj_gemm_kernel(const uint16_t* __restrict__ W, const uint16_t* __restrict__ Phi, const uint16_t* __restrict__ Plo,
                 int64_t M, int N, int K, int NB, int64_t MB, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][3][TILEB];   // [stage][W | Phi | Plo]

  // XCD-aware tile order: the NB feature tiles of one chunk tile run on the same
  // XCD (blocks are dealt round-robin to the 8 XCDs), so its P rows are read once
  // into that XCD's L2.
  const int64_t bid = blockIdx.x;
  const int64_t xcd = bid & 7, slot = bid >> 3;
  const int nb = (int)(slot % NB);
  const int64_t mb = (slot / NB) * 8 + xcd;
  if (mb >= MB) return;
  const int n0 = nb * GT;
  const int64_t m0 = mb * GT;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, hf = lane >> 5;
  const int wn = (wave & 1) * 64, wm = (wave >> 1) * 64;   // this wave's sub-tile

  // global -> register staging: thread t copies rows t/4 and t/4 + 64, 16-byte piece t%4,
  // two stages ahead of the MFMAs (register sets A and B alternate)
  const int srow = tid >> 2, spc = tid & 3;
  int64_t mA = m0 + srow, mB = m0 + srow + 64;
  if (mA >= M) mA = M - 1;                                 // clamp: those chunks are never stored
  if (mB >= M) mB = M - 1;
  const int64_t w0off = (int64_t)(n0 + srow) * K + 8 * spc, w1off = w0off + (int64_t)64 * K;
  const int64_t p0off = mA * K + 8 * spc, p1off = mB * K + 8 * spc;
  struct Stage { uint4 w0, h0, l0, w1, h1, l1; };
  auto fetch = [&](int stage) {
    const int k0 = stage * KS;
    Stage r;
    r.w0 = *reinterpret_cast<const uint4*>(W + w0off + k0);
    r.h0 = *reinterpret_cast<const uint4*>(Phi + p0off + k0);
    r.l0 = *reinterpret_cast<const uint4*>(Plo + p0off + k0);
    r.w1 = *reinterpret_cast<const uint4*>(W + w1off + k0);
    r.h1 = *reinterpret_cast<const uint4*>(Phi + p1off + k0);
    r.l1 = *reinterpret_cast<const uint4*>(Plo + p1off + k0);
    return r;
  };
  auto stash = [&](const Stage& r, int buf) {
    uint8_t* t0 = &lds[buf][0][srow * ROWB + 16 * spc];
    uint8_t* t1 = &lds[buf][0][(srow + 64) * ROWB + 16 * spc];
    *reinterpret_cast<uint4*>(t0) = r.w0;
    *reinterpret_cast<uint4*>(t0 + TILEB) = r.h0;
    *reinterpret_cast<uint4*>(t0 + 2 * TILEB) = r.l0;
    *reinterpret_cast<uint4*>(t1) = r.w1;
    *reinterpret_cast<uint4*>(t1 + TILEB) = r.h1;
    *reinterpret_cast<uint4*>(t1 + 2 * TILEB) = r.l1;
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][c][i] = 0.f;

  auto compute = [&](int buf) {
#pragma unroll
    for (int k16 = 0; k16 < 2; ++k16) {
      const int kb = 32 * k16 + 16 * hf;                   // byte offset of this lane's 8 k values
      bf16x8_t wa[2], ph[2], pl[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        wa[t] = *reinterpret_cast<const bf16x8_t*>(&lds[buf][0][(wn + 32 * t + col) * ROWB + kb]);
        ph[t] = *reinterpret_cast<const bf16x8_t*>(&lds[buf][1][(wm + 32 * t + col) * ROWB + kb]);
        pl[t] = *reinterpret_cast<const bf16x8_t*>(&lds[buf][2][(wm + 32 * t + col) * ROWB + kb]);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[a], ph[c], acc[a][c], 0, 0, 0);
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[a], pl[c], acc[a][c], 0, 0, 0);
        }
    }
  };

  const int nk = K / KS;                                   // >= 1
  // stage s is fetched at most two stages ahead (clamped to the last stage past the end,
  // so every fetch is unconditional and in bounds; the extra copies are never used)
  const int last = nk - 1;
  Stage sa = fetch(0);
  stash(sa, 0);
  sa = fetch(1 < last ? 1 : last);
  Stage sb = fetch(2 < last ? 2 : last);
  __syncthreads();
  for (int ks = 0; ks < nk; ks += 2) {
    // stage ks from buffer 0; stage ks + 1 (set A) goes into buffer 1, read one stage ago
    compute(0);
    if (ks + 1 < nk) stash(sa, 1);
    sa = fetch(ks + 3 < last ? ks + 3 : last);
    __syncthreads();
    if (ks + 1 >= nk) break;
    // stage ks + 1 from buffer 1; stage ks + 2 (set B) into buffer 0
    compute(1);
    if (ks + 2 < nk) stash(sb, 0);
    sb = fetch(ks + 4 < last ? ks + 4 : last);
    __syncthreads();
  }

  // accumulator i of tile (a, c): feature n0 + wn + 32a + 8(i/4) + 4hf + i%4, chunk m0 + wm + 32c + col
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t m = m0 + wm + 32 * c + col;
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int n = n0 + wn + 32 * a + 8 * i4 + 4 * hf;
        const uint32_t w0 = f32_to_bf16_rne(acc[a][c][4 * i4]) | (f32_to_bf16_rne(acc[a][c][4 * i4 + 1]) << 16);
        const uint32_t w1 = f32_to_bf16_rne(acc[a][c][4 * i4 + 2]) | (f32_to_bf16_rne(acc[a][c][4 * i4 + 3]) << 16);
        *reinterpret_cast<uint2*>(out + m * N + n) = make_uint2(w0, w1);
      }
  }
}

}  // namespace

size_t encode_workspace(int64_t n_chunks, int dm) {
  return ((size_t)2 * (size_t)n_chunks * (size_t)dm * sizeof(uint16_t) + 255) & ~(size_t)255;
}

int launch_encode(const uint16_t* hidden, int64_t n_tok, int dm, const uint16_t* W, int N,
                  const int64_t* doc_tok_off, const int64_t* doc_chunk_off, int64_t n_docs, int64_t n_chunks,
                  int chunk_len, uint16_t* Krbar, void* workspace, hipStream_t stream) {
  if (n_chunks == 0) return MSA_OK;
  uint16_t* mean_hi = reinterpret_cast<uint16_t*>(workspace);
  uint16_t* mean_lo = mean_hi + n_chunks * dm;
  const int threads = ((dm / 8 + 63) / 64) * 64;
  hipLaunchKernelGGL(hidden_pool_kernel, dim3((unsigned)n_chunks), dim3(threads), 0, stream, hidden, n_tok, dm,
                     doc_tok_off, doc_chunk_off, n_docs, chunk_len, mean_hi, mean_lo);
  MSA_CHECK_LAUNCH();
  const int NB = N / GT;
  const int64_t MB = (n_chunks + GT - 1) / GT;
  const int64_t blocks = ((MB + 7) / 8) * 8 * NB;
  hipLaunchKernelGGL(proj_gemm_kernel, dim3((unsigned)blocks), dim3(GTHREADS), 0, stream, W, mean_hi, mean_lo,
                     n_chunks, N, dm, NB, MB, Krbar);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

}  // namespace msa
