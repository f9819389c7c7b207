// Chunk-mean pooling with document-wise RoPE (offline Global Memory Encoding).
//
// medium write-up sec. 2 and b-lab.team summary sec. 1: documents are cut
// into fixed-length chunks and K, V and the router key K_r are mean-pooled per
// chunk; b-lab.team sec. 1, Document-wise RoPE: positions restart at 0 in
// every document, so K is rotated at its document-local position before
// pooling.  b-lab.team pipeline stage 1 caches the pooled (Kbar, Vbar, Krbar).
//
// One workgroup per chunk.  The chunk's document comes from a 64-way search of
// the chunk offsets by one wave (3 steps for 200K documents).  The rotation
// table for the chunk's positions is built once per workgroup in LDS with
// fp64 angles.  Each wave accumulates every 4th token in fp32 registers (a lane
// owns 8 dims and their 8 RoPE partners of one head, loaded as 16-byte
// vectors); the four partial sums meet in LDS, and the mean is rounded to bf16
// (nearest even) and stored as 16-byte vectors.  The kernel is HBM-bound:
// 3 * chunk_len * H * D * 2 bytes in, 3 * H * D * 2 bytes out per chunk.
#include "msa_internal.h"

#include <math.h>

namespace msa {
namespace {

constexpr int D = 128;
constexpr int THREADS = 256;
constexpr int MAXC = 64;      // rotation-table rows kept in LDS (longer chunks loop over it)

template <int H>
__global__ void __launch_bounds__(THREADS)
pool_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, const uint16_t* __restrict__ Kr,
            const int64_t* __restrict__ doc_tok_off, const int64_t* __restrict__ doc_chunk_off,
            int64_t n_docs, int64_t n_tok, int64_t n_chunks, int chunk_len, double log2_base,
            uint16_t* __restrict__ Kbar, uint16_t* __restrict__ Vbar, uint16_t* __restrict__ Krbar) {
  constexpr int LANES_PER_TOK = H * 8;                 // lane -> (head, 8-dim group)
  constexpr int TOKPAR = THREADS / LANES_PER_TOK;      // tokens in flight per step
  __shared__ float cs_tab[MAXC][D / 2];
  __shared__ float sn_tab[MAXC][D / 2];
  __shared__ float part[TOKPAR][3][H * D];
  __shared__ int64_t sh_doc;

  const int tid = threadIdx.x;
  const int64_t gl = blockIdx.x;                       // local chunk row
  const int64_t cbase = doc_chunk_off[0];
  const int64_t g = cbase + gl;                        // global chunk index

  // --- find the document: doc_chunk_off[d] <= g < doc_chunk_off[d+1]
  if (tid < 64) {
    int64_t lo = 0, hi = n_docs;
    while (hi - lo > 1) {
      const int64_t span = hi - lo;
      const int64_t piv = lo + (span * tid) / 64;
      const bool le = doc_chunk_off[piv] <= g;
      const uint64_t mask = __ballot(le);
      const int c = __popcll(mask);                    // pivots at or below g form a prefix
      const int64_t nlo = lo + (span * (c - 1)) / 64;
      const int64_t nhi = (c < 64) ? lo + (span * c) / 64 : hi;
      lo = nlo;
      hi = nhi > nlo ? nhi : nlo + 1;
    }
    if (tid == 0) sh_doc = lo;
  }
  __syncthreads();
  const int64_t d = sh_doc;
  const int64_t j = g - doc_chunk_off[d];
  const int64_t tbase = doc_tok_off[0];
  const int64_t doc_t0 = doc_tok_off[d];
  const int64_t L = doc_tok_off[d + 1] - doc_t0;
  const int64_t p0 = j * chunk_len;                    // first document-local position
  int cnt = (int)((L - p0) < chunk_len ? (L - p0) : chunk_len);
  const int64_t row0 = doc_t0 - tbase + p0;            // first input row
  if (cnt < 0 || row0 < 0 || row0 + cnt > n_tok) cnt = 0;   // inconsistent offsets: write zeros

  const int tq = tid / LANES_PER_TOK;                  // token phase of this lane
  const int ln = tid % LANES_PER_TOK;
  const int h = ln / 8, grp = ln % 8;
  const int i0 = grp * 8;                              // pair indices i0..i0+7 (dims i and i+64)
  float ak[16], av[16], ar[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) { ak[e] = 0.f; av[e] = 0.f; ar[e] = 0.f; }

  for (int t0 = 0; t0 < cnt; t0 += MAXC) {
    const int tn = (cnt - t0) < MAXC ? (cnt - t0) : MAXC;
    __syncthreads();
    for (int x = tid; x < tn * (D / 2); x += THREADS) {
      const int tt = x / (D / 2), i = x % (D / 2);
      const double theta = exp2(-(2.0 * i / D) * log2_base);
      double sn, cs;
      sincos((double)(p0 + t0 + tt) * theta, &sn, &cs);
      cs_tab[tt][i] = (float)cs;
      sn_tab[tt][i] = (float)sn;
    }
    __syncthreads();
    for (int tt = tq; tt < tn; tt += TOKPAR) {
      const int64_t r = row0 + t0 + tt;
      const int64_t base = (r * H + h) * D;
      const uint4 k1 = load_nt16(K + base + i0);          // raw tokens are read once
      const uint4 k2 = load_nt16(K + base + 64 + i0);
      const uint4 v1 = load_nt16(V + base + i0);
      const uint4 v2 = load_nt16(V + base + 64 + i0);
      const uint4 r1 = load_nt16(Kr + base + i0);
      const uint4 r2 = load_nt16(Kr + base + 64 + i0);
      const uint32_t kw1[4] = {k1.x, k1.y, k1.z, k1.w}, kw2[4] = {k2.x, k2.y, k2.z, k2.w};
      const uint32_t vw1[4] = {v1.x, v1.y, v1.z, v1.w}, vw2[4] = {v2.x, v2.y, v2.z, v2.w};
      const uint32_t rw1[4] = {r1.x, r1.y, r1.z, r1.w}, rw2[4] = {r2.x, r2.y, r2.z, r2.w};
      const float4 c0 = *reinterpret_cast<const float4*>(&cs_tab[tt][i0]);
      const float4 c1 = *reinterpret_cast<const float4*>(&cs_tab[tt][i0 + 4]);
      const float4 s0 = *reinterpret_cast<const float4*>(&sn_tab[tt][i0]);
      const float4 s1 = *reinterpret_cast<const float4*>(&sn_tab[tt][i0 + 4]);
      const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w1 = kw1[e >> 1], w2 = kw2[e >> 1];
        const float x1 = (e & 1) ? bf16_hi(w1) : bf16_lo(w1);
        const float x2 = (e & 1) ? bf16_hi(w2) : bf16_lo(w2);
        ak[e] += x1 * cc[e] - x2 * ss[e];
        ak[8 + e] += x2 * cc[e] + x1 * ss[e];
        av[e] += (e & 1) ? bf16_hi(vw1[e >> 1]) : bf16_lo(vw1[e >> 1]);
        av[8 + e] += (e & 1) ? bf16_hi(vw2[e >> 1]) : bf16_lo(vw2[e >> 1]);
        ar[e] += (e & 1) ? bf16_hi(rw1[e >> 1]) : bf16_lo(rw1[e >> 1]);
        ar[8 + e] += (e & 1) ? bf16_hi(rw2[e >> 1]) : bf16_lo(rw2[e >> 1]);
      }
    }
  }

  // --- combine the TOKPAR token phases, divide, round, store
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    part[tq][0][h * D + i0 + e] = ak[e];
    part[tq][0][h * D + 64 + i0 + e] = ak[8 + e];
    part[tq][1][h * D + i0 + e] = av[e];
    part[tq][1][h * D + 64 + i0 + e] = av[8 + e];
    part[tq][2][h * D + i0 + e] = ar[e];
    part[tq][2][h * D + 64 + i0 + e] = ar[8 + e];
  }
  __syncthreads();
  if (gl >= n_chunks) return;
  const float inv = cnt > 0 ? 1.0f / (float)cnt : 0.f;
  constexpr int VEC = 3 * H * D / 8;                   // 16-byte output vectors
  for (int x = tid; x < VEC; x += THREADS) {
    const int which = x / (H * D / 8);
    const int col = (x % (H * D / 8)) * 8;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int p = 0; p < TOKPAR; ++p) {
        a0 += part[p][which][col + 2 * e];
        a1 += part[p][which][col + 2 * e + 1];
      }
      w[e] = f32_to_bf16_rne(a0 * inv) | (f32_to_bf16_rne(a1 * inv) << 16);
    }
    uint16_t* dst = (which == 0 ? Kbar : which == 1 ? Vbar : Krbar) + gl * (int64_t)(H * D) + col;
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

int launch_pool(const uint16_t* K, const uint16_t* V, const uint16_t* Kr, const int64_t* doc_tok_off,
                const int64_t* doc_chunk_off, int64_t n_docs, int64_t n_tok, int64_t n_chunks, int H,
                int chunk_len, double rope_base, uint16_t* Kbar, uint16_t* Vbar, uint16_t* Krbar,
                hipStream_t stream) {
  if (n_chunks == 0) return MSA_OK;
  const double lb = log2(rope_base);
  dim3 grid((unsigned)n_chunks);
#define MSA_POOL_CASE(HH)                                                                        \
  case HH:                                                                                       \
    hipLaunchKernelGGL(pool_kernel<HH>, grid, dim3(THREADS), 0, stream, K, V, Kr, doc_tok_off,  \
                       doc_chunk_off, n_docs, n_tok, n_chunks, chunk_len, lb, Kbar, Vbar, Krbar); \
    break;
  switch (H) {
    MSA_POOL_CASE(1)
    MSA_POOL_CASE(2)
    MSA_POOL_CASE(4)
    MSA_POOL_CASE(8)
    MSA_POOL_CASE(16)
    default: set_error("H=%d unsupported", H); return MSA_ERR_UNSUPPORTED;
  }
#undef MSA_POOL_CASE
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

}  // namespace msa
