// Chunk-mean pooling with document-wise RoPE (offline Global Memory Encoding).
//
// medium write-up sec. 2 and b-lab.team summary sec. 1: documents are cut
// into fixed-length chunks and K, V and the router key K_r are mean-pooled per
// chunk; b-lab.team sec. 1, Document-wise RoPE: positions restart at 0 in
// every document, so K is rotated at its document-local position before
// pooling.  b-lab.team pipeline stage 1 caches the pooled (Kbar, Vbar, Krbar).
//
// The step is a streaming reduction bound by HBM (3 * chunk_len * H * D * 2
// bytes in, 3 * H * D * 2 bytes out per chunk), so the kernel is laid out to
// keep many independent loads in flight and to touch LDS as little as possible:
//
//  * A workgroup is four waves walking the workgroup's contiguous range of
//    chunks as a list of (chunk, tensor) items, tensor = K, V, K_r in turn;
//    wave w takes items w, w + 4, ..., so the rotation work of K is shared
//    evenly (a wave that always took K lagged those that only add).  A wave
//    keeps an item's sums in registers (a lane owns 8 dims of a head and their
//    8 RoPE partners, read as 16-byte non-temporal loads, 16 tokens per step),
//    so no partial sums meet in LDS and the waves never wait for one another.
//  * Rotation is linear, so a chunk's rotated sum is
//      sum_t R((p0 + t) theta) K_t = R(p0 theta) sum_t R(t theta) K_t :
//    the wave holding K rotates every token by its offset t inside the chunk, from a
//    table of cos/sin(t theta_i), t < 64, built once per workgroup in LDS
//    (angles reduced in fp64), and rotates the finished sum once by the chunk's
//    start angle (longer chunks do this per block of 64 tokens).
//  * The chunk's document is found once per workgroup by a 64-way search of
//    the chunk offsets and then advanced chunk by chunk.
// The three sums are divided by the token count, rounded to bf16 (nearest
// even) and stored as 16-byte vectors.
#include "msa_internal.h"

#include <math.h>

namespace msa {
namespace {

constexpr int D = 128;
constexpr int TABT = 64;           // token offsets in the rotation table (one block)
constexpr int WG_PER_CU = 2;       // four waves of ~230 registers each: two workgroups per CU
constexpr int STEP = 16;           // tokens per load batch
constexpr int POOL_WAVES = 4;      // waves per workgroup

// Lane layout for H heads: a token row of one tensor is H * D bf16; a lane takes 8 dims
// [i0, i0 + 8) of a head and their partners [64 + i0, 72 + i0).  With H < 8 a wave covers
// TPW = 8 / H tokens at once; with H = 16 a lane takes two heads.
template <int H>
struct PoolCfg {
  static constexpr int TPW = H >= 8 ? 1 : 8 / H;   // tokens per wave step
  static constexpr int HPL = H >= 8 ? H / 8 : 1;   // heads per lane
};

// First chunk of document d and the document of chunk g (doc_chunk_off[d] <= g < doc_chunk_off[d+1]),
// by one wave: 64 pivots per step narrow [lo, hi) by 64x.
__device__ int64_t find_doc(const int64_t* __restrict__ doc_chunk_off, int64_t n_docs, int64_t g, int lane) {
  int64_t lo = 0, hi = n_docs;
  while (hi - lo > 1) {
    const int64_t span = hi - lo;
    const int64_t piv = lo + (span * lane) / 64;
    const bool le = doc_chunk_off[piv] <= g;
    const uint64_t mask = __ballot(le);
    const int c = __popcll(mask);                        // pivots at or below g form a prefix
    const int64_t nlo = lo + (span * (c - 1)) / 64;
    const int64_t nhi = (c < 64) ? lo + (span * c) / 64 : hi;
    lo = nlo;
    hi = nhi > nlo ? nhi : nlo + 1;
  }
  return lo;
}

// 8 bf16 (one 16-byte load) -> fp32, added to acc[0..8)
__device__ __forceinline__ void add8(const uint4 v, float* acc) {
  acc[0] += bf16_lo(v.x); acc[1] += bf16_hi(v.x);
  acc[2] += bf16_lo(v.y); acc[3] += bf16_hi(v.y);
  acc[4] += bf16_lo(v.z); acc[5] += bf16_hi(v.z);
  acc[6] += bf16_lo(v.w); acc[7] += bf16_hi(v.w);
}

// The rotated pair sum: a1 += x1 c - x2 s, a2 += x2 c + x1 s for 8 frequencies.
__device__ __forceinline__ void rot_add8(const uint4 u1, const uint4 u2, const float2* __restrict__ cs, float* a1,
                                         float* a2) {
  const uint32_t w1[4] = {u1.x, u1.y, u1.z, u1.w}, w2[4] = {u2.x, u2.y, u2.z, u2.w};
  const float4 t0 = *reinterpret_cast<const float4*>(cs);
  const float4 t1 = *reinterpret_cast<const float4*>(cs + 2);
  const float4 t2 = *reinterpret_cast<const float4*>(cs + 4);
  const float4 t3 = *reinterpret_cast<const float4*>(cs + 6);
  const float c[8] = {t0.x, t0.z, t1.x, t1.z, t2.x, t2.z, t3.x, t3.z};
  const float s[8] = {t0.y, t0.w, t1.y, t1.w, t2.y, t2.w, t3.y, t3.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x1 = (e & 1) ? bf16_hi(w1[e >> 1]) : bf16_lo(w1[e >> 1]);
    const float x2 = (e & 1) ? bf16_hi(w2[e >> 1]) : bf16_lo(w2[e >> 1]);
    a1[e] = fmaf(x1, c[e], a1[e]);
    a1[e] = fmaf(-x2, s[e], a1[e]);
    a2[e] = fmaf(x2, c[e], a2[e]);
    a2[e] = fmaf(x1, s[e], a2[e]);
  }
}

struct ChunkInfo {
  int64_t row0;    // first input row
  int64_t p0;      // document-local position of the first token
  int cnt;         // tokens (0 when the offsets are inconsistent: the chunk is written as zeros)
};

template <int H>
__global__ void __launch_bounds__(64 * POOL_WAVES)
pool_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, const uint16_t* __restrict__ Kr,
            const int64_t* __restrict__ doc_tok_off, const int64_t* __restrict__ doc_chunk_off,
            int64_t n_docs, int64_t n_tok, int64_t n_chunks, int64_t per_wg, int chunk_len, double log2_base,
            uint16_t* __restrict__ Kbar, uint16_t* __restrict__ Vbar, uint16_t* __restrict__ Krbar) {
  using CF = PoolCfg<H>;
  // cos/sin(t theta_i), t < 64, i < 64, as (cos, sin) pairs; rows padded by 16 bytes so that
  // lanes reading different t rows at the same i fall in different banks
  __shared__ __attribute__((aligned(16))) float2 tab[TABT][D / 2 + 2];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t c_begin = (int64_t)blockIdx.x * per_wg;
  int64_t c_end = c_begin + per_wg;
  if (c_end > n_chunks) c_end = n_chunks;

  // rotation table (angles reduced in fp64, evaluated in fp32)
  for (int x = threadIdx.x; x < TABT * (D / 2); x += 64 * POOL_WAVES) {
    const int t = x / (D / 2), i = x % (D / 2);
    const double rev = exp2(-(2.0 * i / D) * log2_base) * 0.15915494309189535;   // theta_i / (2 pi)
    float c, s;
    rope_cs(t, rev, &c, &s);
    tab[t][i] = make_float2(c, s);
  }
  __syncthreads();
  if (c_begin >= c_end) return;

  const int ln = lane % (8 * H < 64 ? 8 * H : 64);
  const int tsub = lane / (8 * H < 64 ? 8 * H : 64);         // token sub-index (H < 8)
  const int grp = ln % 8;                                     // 8-dim group: pair dims i0..i0+7
  const int h0 = ln / 8;                                      // first head of the lane
  const int i0 = grp * 8;
  double rev[8];                                              // this lane's frequencies, for the start angles
#pragma unroll
  for (int e = 0; e < 8; ++e) rev[e] = exp2(-(2.0 * (i0 + e) / D) * log2_base) * 0.15915494309189535;

  const int64_t cbase = doc_chunk_off[0];
  const int64_t tbase = doc_tok_off[0];
  int64_t d = find_doc(doc_chunk_off, n_docs, cbase + c_begin, lane);
  const int64_t n_items = 3 * (c_end - c_begin);
  for (int64_t j = wave; j < n_items; j += POOL_WAVES) {
    const int64_t gl = c_begin + j / 3;
    const int64_t g = cbase + gl;
    const int role = (int)(j % 3);                              // 0: K, 1: V, 2: K_r
    const uint16_t* src = role == 0 ? K : (role == 1 ? V : Kr);
    uint16_t* dst = role == 0 ? Kbar : (role == 1 ? Vbar : Krbar);
    while (d + 1 < n_docs && doc_chunk_off[d + 1] <= g) ++d;
    ChunkInfo ci;
    {
      const int64_t doc_t0 = doc_tok_off[d];
      const int64_t L = doc_tok_off[d + 1] - doc_t0;
      ci.p0 = (g - doc_chunk_off[d]) * chunk_len;
      int64_t cnt = L - ci.p0 < chunk_len ? L - ci.p0 : chunk_len;
      ci.row0 = doc_t0 - tbase + ci.p0;
      if (cnt < 0 || ci.row0 < 0 || ci.row0 + cnt > n_tok || g < doc_chunk_off[d]) cnt = 0;
      ci.cnt = (int)cnt;
    }
    float out1[CF::HPL][8], out2[CF::HPL][8];                // the chunk's sums (dims i0.., 64 + i0..)
#pragma unroll
    for (int hp = 0; hp < CF::HPL; ++hp)
#pragma unroll
      for (int e = 0; e < 8; ++e) { out1[hp][e] = 0.f; out2[hp][e] = 0.f; }

    for (int b0 = 0; b0 < ci.cnt; b0 += TABT) {              // blocks of 64 tokens
      const int bn = ci.cnt - b0 < TABT ? ci.cnt - b0 : TABT;
      float a1[CF::HPL][8], a2[CF::HPL][8];
#pragma unroll
      for (int hp = 0; hp < CF::HPL; ++hp)
#pragma unroll
        for (int e = 0; e < 8; ++e) { a1[hp][e] = 0.f; a2[hp][e] = 0.f; }
      for (int t0 = 0; t0 < bn; t0 += STEP * CF::TPW) {
        uint4 u1[STEP][CF::HPL], u2[STEP][CF::HPL];
#pragma unroll
        for (int k = 0; k < STEP; ++k) {
          const int t = t0 + k * CF::TPW + tsub;
#pragma unroll
          for (int hp = 0; hp < CF::HPL; ++hp) {
            u1[k][hp] = make_uint4(0, 0, 0, 0);
            u2[k][hp] = make_uint4(0, 0, 0, 0);
            if (t < bn) {
              const uint16_t* p = src + ((ci.row0 + b0 + t) * H + h0 + 8 * hp) * D + i0;
              u1[k][hp] = load_nt16(p);                         // raw tokens are read once
              u2[k][hp] = load_nt16(p + 64);
            }
          }
        }
#pragma unroll
        for (int k = 0; k < STEP; ++k) {
          const int t = t0 + k * CF::TPW + tsub;
          if (role == 0) {
            const float2* cs = &tab[t < TABT ? t : 0][i0];      // zero rows past bn add nothing
#pragma unroll
            for (int hp = 0; hp < CF::HPL; ++hp) rot_add8(u1[k][hp], u2[k][hp], cs, a1[hp], a2[hp]);
          } else {
#pragma unroll
            for (int hp = 0; hp < CF::HPL; ++hp) { add8(u1[k][hp], a1[hp]); add8(u2[k][hp], a2[hp]); }
          }
        }
      }
      if (role == 0) {
        // rotate the block's sum by its first token's angle, R((p0 + b0) theta)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float c, s;
          rope_cs((int)(ci.p0 + b0), rev[e], &c, &s);
#pragma unroll
          for (int hp = 0; hp < CF::HPL; ++hp) {
            out1[hp][e] += a1[hp][e] * c - a2[hp][e] * s;
            out2[hp][e] += a2[hp][e] * c + a1[hp][e] * s;
          }
        }
      } else {
#pragma unroll
        for (int hp = 0; hp < CF::HPL; ++hp)
#pragma unroll
          for (int e = 0; e < 8; ++e) { out1[hp][e] += a1[hp][e]; out2[hp][e] += a2[hp][e]; }
      }
    }
    // H < 8: add the token sub-lanes' sums (lanes 8H, 16H, ... apart), in a fixed order
#pragma unroll
    for (int m = 8 * H; m < 64; m <<= 1) {
#pragma unroll
      for (int hp = 0; hp < CF::HPL; ++hp)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          out1[hp][e] += __shfl_xor(out1[hp][e], m);
          out2[hp][e] += __shfl_xor(out2[hp][e], m);
        }
    }
    if (tsub == 0) {
      const float inv = ci.cnt > 0 ? 1.0f / (float)ci.cnt : 0.f;
#pragma unroll
      for (int hp = 0; hp < CF::HPL; ++hp) {
        uint16_t* o = dst + (gl * H + h0 + 8 * hp) * D + i0;
        uint32_t w1[4], w2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w1[e] = f32_to_bf16_rne(out1[hp][2 * e] * inv) | (f32_to_bf16_rne(out1[hp][2 * e + 1] * inv) << 16);
          w2[e] = f32_to_bf16_rne(out2[hp][2 * e] * inv) | (f32_to_bf16_rne(out2[hp][2 * e + 1] * inv) << 16);
        }
        *reinterpret_cast<uint4*>(o) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
        *reinterpret_cast<uint4*>(o + 64) = make_uint4(w2[0], w2[1], w2[2], w2[3]);
      }
    }
  }
}

}  // namespace

int launch_pool(const uint16_t* K, const uint16_t* V, const uint16_t* Kr, const int64_t* doc_tok_off,
                const int64_t* doc_chunk_off, int64_t n_docs, int64_t n_tok, int64_t n_chunks, int H,
                int chunk_len, double rope_base, uint16_t* Kbar, uint16_t* Vbar, uint16_t* Krbar,
                hipStream_t stream) {
  if (n_chunks == 0) return MSA_OK;
  const double lb = log2(rope_base);
  int64_t wgs = (int64_t)num_cus() * WG_PER_CU;
  if (wgs > n_chunks) wgs = n_chunks;
  const int64_t per = (n_chunks + wgs - 1) / wgs;
  wgs = (n_chunks + per - 1) / per;
  dim3 grid((unsigned)wgs);
#define MSA_POOL_CASE(HH)                                                                        \
  case HH:                                                                                       \
    hipLaunchKernelGGL(pool_kernel<HH>, grid, dim3(64 * POOL_WAVES), 0, stream, K, V, Kr, doc_tok_off,       \
                       doc_chunk_off, n_docs, n_tok, n_chunks, per, chunk_len, lb, Kbar, Vbar, Krbar); \
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
