// Backward of the sparse attention over [pooled memory ++ causal local KV]: the
// gradients of Q, the local K and V, and the selected documents' pooled K and V,
// given dL/dO.
//
// chatpaper.ai Abstract: MSA is trained end to end, so the loss reaches the
// query, the local context and the retrieved memory through this attention;
// medium write-up sec. 2 and b-lab.team summary sec. 1 define the forward
// (memory K/V concatenated with the local K/V, Global RoPE offset k).  Per
// q-head, S = scale * Qrot Krot^T (masked), P = softmax_rows(S), O = P V:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Delta),  Delta_i = sum_j P_ij dP_ij,
//   dQrot = scale * dS K,  dK = scale * dS^T Qrot,
// a kv-head collects the gradients of its q-heads, and the gradient of a rotated
// input is rotated back (the rotation is orthogonal).  Memory keys are used as
// given, so their gradient is taken as is.
//
// Kernels, in launch order:
//   bwd_prep_kernel   one 32-row (or 32-key) tile per workgroup: rotate Q
//       and the local keys, split every fp32 operand into bf16 hi + lo parts
//       (x = hi + lo, |lo| <= 2^-9 |x|) and lay the operands out per head,
//       row-major and transposed (through an LDS tile, 16-byte stores), padded
//       to 32-row / 32-key tiles with zeros; keys in the forward's order
//       (memory, then local)
//   bwd_stats_kernel  32 query rows of one q-head per workgroup; the 4 waves
//       take every 4th key tile: row max, sum and Delta online (S^T = K Q^T and
//       dP^T = V dO^T on v_mfma_f32_32x32x16_bf16, one query row per lane pair),
//       merged over the waves -> log2-sum-exp and Delta per row
//   bwd_grad_kernel  one launch, two kinds of workgroup that run side by side:
//       query side (32 rows of one q-head): dS^T per tile and dQ += dS K with
//       the key dimension as the contraction; key side (32 keys of one kv-head,
//       their K and V rows resident as B operands, the waves splitting the
//       (q-head, row tile) pairs): S = Q K^T and dP = dO V^T give P and dS with
//       one key per lane pair, then dV += P^T dO and dK += dS^T Qrot with the row
//       dimension as the contraction (transposed dO and Qrot from the prep).
// Every product uses the split operands (hi*hi + hi*lo + lo*hi; two products
// where one side is an exact bf16 input), so with fp32 accumulation the
// gradients keep ~2^-16 relative accuracy.  The waves' partial results are
// added in a fixed order: no atomics, results independent of scheduling.
#include "msa_internal.h"

#include <math.h>

namespace msa {
namespace {

constexpr int D = 128;
constexpr int NW = 4;
constexpr int THREADS = 64 * NW;
constexpr int PSTRIDE = D + 4;     // floats per (wave, row) in the merge area
// q-heads per key-side workgroup: one (its waves each take one row tile at the step's
// shape); two per workgroup halves the launch but measured slower
constexpr int KV_HPW = 1;

struct RopeRev {
  double rev[D / 2];               // theta_i / (2 pi)
};

__device__ __forceinline__ uint16_t bf16_bits(float x) { return (uint16_t)f32_to_bf16_rne(x); }
__device__ __forceinline__ float bits_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// hi + lo split of 8 fp32 values into two bf16x8 operands
__device__ __forceinline__ void split8(const float* x, bf16x8_t& hi, bf16x8_t& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = cvt2_bf16(x[2 * e], x[2 * e + 1]);
    l[e] = cvt2_bf16(x[2 * e] - bf16_lo(h[e]), x[2 * e + 1] - bf16_hi(h[e]));
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

__device__ __forceinline__ bf16x8_t ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}
// Transposed operands (the B side of products whose contraction runs over rows or
// keys) are stored in blocks of 16 rows: [block][dim][16], the 16 rows of a block in
// the order rows {0..3, 8..11, 4..7, 12..15}.  A lane with half index hf holds rows
// {4 hf .. 4 hf + 3, 8 + 4 hf .. 8 + 4 hf + 3} of an MFMA result, so its 8 B-operand
// values are stored positions 8 hf .. 8 hf + 7: one 16-byte load, and the 64 lanes
// of a wave read 1 KB of contiguous memory.
__device__ __forceinline__ int blk_row(int j) { return (j & 3) | ((j & 4) << 1) | ((j & 8) >> 1); }

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int clamp_mem(const int32_t* mem_len, int b, int Mmax) {
  int M = mem_len[b];
  return M < 0 ? 0 : (M > Mmax ? Mmax : M);
}

constexpr int TS = D + 8;          // LDS transpose tile row stride (bf16): 16-byte rows, banks staggered

__device__ __forceinline__ void unpack8(uint4 v, float* x) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}
__device__ __forceinline__ uint4 u4(bf16x8_t v) { return __builtin_bit_cast(uint4, v); }

// Rotate 8 pairs (x1[e], x2[e]) = dims (p0 + e, p0 + 64 + e) at position pos.
__device__ __forceinline__ void rotate8(float* x1, float* x2, int pos, const RopeRev& rr, int p0) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float c, s;
    rope_cs(pos, rr.rev[p0 + e], &c, &s);
    const float a = x1[e], b = x2[e];
    x1[e] = a * c - b * s;
    x2[e] = b * c + a * s;
  }
}

// Stored positions 8 hf .. 8 hf + 7 of the 16-row block starting at row r0 of an LDS
// tile, dim d: 16 bytes of the blocked transposed layout.
__device__ __forceinline__ uint4 tile_blk8(const uint16_t (*t)[TS], int r0, int hf, int d) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = (uint32_t)t[r0 + blk_row(8 * hf + 2 * e)][d] | ((uint32_t)t[r0 + blk_row(8 * hf + 2 * e + 1)][d] << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// 32 query rows of one q-head: Q rotated at rope_offset + (Tl - Tq) + i and split,
// dO split.  Row-major [B, Hq, Tq32, D] (16-byte stores) and transposed
// [B, Hq, Tq32 / 16, D, 16] (16-row blocks, see blk_row) through an LDS tile; rows
// >= Tq are zeros.
struct PrepArgs {
  const uint16_t *Q, *Kloc, *Vloc, *Kmem, *Vmem;
  const float* dO;
  const float *O, *lse;   // the forward's output and natural log-sum-exp [B, Tq, Hq], or null
  float *LSE2, *DLT;      // per-row statistics the gradient pass reads (written here when O is given)
  const int32_t* mem_len;
  int B, Tq, Tq32, Hq, Tl, Hkv, Mmax, NK, rope_offset;
  int64_t mstride;
  uint16_t *Qh, *Ql, *QTh, *QTl, *Oh, *Ol, *OTh, *OTl, *Kh, *Kl, *KTh, *KTl, *Vc;
  float *dKmem, *dVmem;
};

__device__ __forceinline__ void prep_q_tile(const uint16_t* __restrict__ Q, const float* __restrict__ dO, int Tq,
                                            int Tq32, int Hq, int Tl, int rope_offset, const RopeRev& rr,
                                            uint16_t* __restrict__ Qh, uint16_t* __restrict__ Ql,
                                            uint16_t* __restrict__ QTh, uint16_t* __restrict__ QTl,
                                            uint16_t* __restrict__ Oh, uint16_t* __restrict__ Ol,
                                            uint16_t* __restrict__ OTh, uint16_t* __restrict__ OTl, int rt, int h,
                                            int b, uint16_t (*tile)[32][TS], const float* __restrict__ Ofw,
                                            const float* __restrict__ lse, float* __restrict__ LSE2,
                                            float* __restrict__ DLT) {
  const int tid = threadIdx.x;
  const int r = tid >> 3, p0 = (tid & 7) * 8;                           // tile row, first pair
  const int i = rt * 32 + r;
  float q1[8], q2[8], o1[8], o2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q1[e] = q2[e] = o1[e] = o2[e] = 0.f;
  if (i < Tq) {
    const int64_t src = (((int64_t)b * Tq + i) * Hq + h) * D;
    unpack8(*reinterpret_cast<const uint4*>(Q + src + p0), q1);
    unpack8(*reinterpret_cast<const uint4*>(Q + src + 64 + p0), q2);
    const float4 a0 = *reinterpret_cast<const float4*>(dO + src + p0);
    const float4 a1 = *reinterpret_cast<const float4*>(dO + src + p0 + 4);
    const float4 b0 = *reinterpret_cast<const float4*>(dO + src + 64 + p0);
    const float4 b1 = *reinterpret_cast<const float4*>(dO + src + 64 + p0 + 4);
    o1[0] = a0.x; o1[1] = a0.y; o1[2] = a0.z; o1[3] = a0.w; o1[4] = a1.x; o1[5] = a1.y; o1[6] = a1.z; o1[7] = a1.w;
    o2[0] = b0.x; o2[1] = b0.y; o2[2] = b0.z; o2[3] = b0.w; o2[4] = b1.x; o2[5] = b1.y; o2[6] = b1.z; o2[7] = b1.w;
    rotate8(q1, q2, rope_offset + (Tl - Tq) + i, rr, p0);
  }
  // With the forward's output and log-sum-exp: Delta_i = sum_d dO_id O_id (= sum_j P_ij dP_ij)
  // and the log2-sum-exp of the pre-scaled scores, so the statistics pass is not needed.
  // The 8 threads of a row are consecutive lanes of one wave.
  if (Ofw) {
    float dl = 0.f;
    if (i < Tq) {
      const int64_t src = (((int64_t)b * Tq + i) * Hq + h) * D;
      const float4 c0 = *reinterpret_cast<const float4*>(Ofw + src + p0);
      const float4 c1 = *reinterpret_cast<const float4*>(Ofw + src + p0 + 4);
      const float4 d0 = *reinterpret_cast<const float4*>(Ofw + src + 64 + p0);
      const float4 d1 = *reinterpret_cast<const float4*>(Ofw + src + 64 + p0 + 4);
      dl = o1[0] * c0.x + o1[1] * c0.y + o1[2] * c0.z + o1[3] * c0.w + o1[4] * c1.x + o1[5] * c1.y + o1[6] * c1.z +
           o1[7] * c1.w + o2[0] * d0.x + o2[1] * d0.y + o2[2] * d0.z + o2[3] * d0.w + o2[4] * d1.x + o2[5] * d1.y +
           o2[6] * d1.z + o2[7] * d1.w;
    }
    dl += __shfl_xor(dl, 1);
    dl += __shfl_xor(dl, 2);
    dl += __shfl_xor(dl, 4);
    if ((tid & 7) == 0) {
      const int64_t st = ((int64_t)b * Hq + h) * Tq32 + i;
      DLT[st] = i < Tq ? dl : 0.f;
      LSE2[st] = i < Tq ? lse[((int64_t)b * Tq + i) * Hq + h] * 1.4426950408889634f : INFINITY;   // padded rows: P = 0
    }
  }
  bf16x8_t qh1, ql1, qh2, ql2, oh1, ol1, oh2, ol2;
  split8(q1, qh1, ql1);
  split8(q2, qh2, ql2);
  split8(o1, oh1, ol1);
  split8(o2, oh2, ol2);
  const int64_t row = (((int64_t)b * Hq + h) * Tq32 + i) * D;
  *reinterpret_cast<uint4*>(Qh + row + p0) = u4(qh1); *reinterpret_cast<uint4*>(Qh + row + 64 + p0) = u4(qh2);
  *reinterpret_cast<uint4*>(Ql + row + p0) = u4(ql1); *reinterpret_cast<uint4*>(Ql + row + 64 + p0) = u4(ql2);
  *reinterpret_cast<uint4*>(Oh + row + p0) = u4(oh1); *reinterpret_cast<uint4*>(Oh + row + 64 + p0) = u4(oh2);
  *reinterpret_cast<uint4*>(Ol + row + p0) = u4(ol1); *reinterpret_cast<uint4*>(Ol + row + 64 + p0) = u4(ol2);
  *reinterpret_cast<uint4*>(&tile[0][r][p0]) = u4(qh1); *reinterpret_cast<uint4*>(&tile[0][r][64 + p0]) = u4(qh2);
  *reinterpret_cast<uint4*>(&tile[1][r][p0]) = u4(ql1); *reinterpret_cast<uint4*>(&tile[1][r][64 + p0]) = u4(ql2);
  *reinterpret_cast<uint4*>(&tile[2][r][p0]) = u4(oh1); *reinterpret_cast<uint4*>(&tile[2][r][64 + p0]) = u4(oh2);
  *reinterpret_cast<uint4*>(&tile[3][r][p0]) = u4(ol1); *reinterpret_cast<uint4*>(&tile[3][r][64 + p0]) = u4(ol2);
  __syncthreads();
  // transposed blocks: (array, 16-row block, dim, half), 16 bytes each
  uint16_t* const dst[4] = {QTh, QTl, OTh, OTl};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int id = tid + 256 * k;
    const int a = id >> 9, rb = (id >> 8) & 1, d = (id >> 1) & (D - 1), hf = id & 1;
    const int64_t blk = ((int64_t)b * Hq + h) * (Tq32 / 16) + rt * 2 + rb;
    *reinterpret_cast<uint4*>(dst[a] + (blk * D + d) * 16 + 8 * hf) = tile_blk8(tile[a], 16 * rb, hf, d);
  }
}

// 32 keys of one kv-head in the forward's order (memory entries, then local keys
// rotated at rope_offset + j), split; row-major [B, Hkv, NK, D], transposed
// [B, Hkv, NK / 16, D, 16] through an LDS tile, V row-major (exact bf16).  Keys >= M + Tl are
// zeros.  Also zeroes the memory-gradient entries [M, Mmax).
__device__ __forceinline__ void prep_k_tile(const uint16_t* __restrict__ Kloc, const uint16_t* __restrict__ Vloc,
                                            int Tl, int Hkv, const uint16_t* __restrict__ Kmem,
                                            const uint16_t* __restrict__ Vmem, int64_t mstride, int Mmax,
                                            const int32_t* __restrict__ mem_len, int NK, int rope_offset,
                                            const RopeRev& rr, uint16_t* __restrict__ Kh, uint16_t* __restrict__ Kl,
                                            uint16_t* __restrict__ KTh, uint16_t* __restrict__ KTl,
                                            uint16_t* __restrict__ Vc, float* __restrict__ dKmem,
                                            float* __restrict__ dVmem, int kt, int g, int b,
                                            uint16_t (*tile)[32][TS]) {
  const int tid = threadIdx.x;
  const int r = tid >> 3, p0 = (tid & 7) * 8;
  const int kk = kt * 32 + r;
  const int M = clamp_mem(mem_len, b, Mmax);
  uint4 kh1 = make_uint4(0, 0, 0, 0), kh2 = kh1, kl1 = kh1, kl2 = kh1, v1 = kh1, v2 = kh1;
  if (kk < M) {
    const int64_t e = ((int64_t)b * Mmax + kk) * mstride + (int64_t)g * D;
    kh1 = *reinterpret_cast<const uint4*>(Kmem + e + p0);
    kh2 = *reinterpret_cast<const uint4*>(Kmem + e + 64 + p0);
    v1 = *reinterpret_cast<const uint4*>(Vmem + e + p0);
    v2 = *reinterpret_cast<const uint4*>(Vmem + e + 64 + p0);
  } else if (kk < M + Tl) {
    const int j = kk - M;
    const int64_t e = (((int64_t)b * Tl + j) * Hkv + g) * D;
    float k1[8], k2[8];
    unpack8(*reinterpret_cast<const uint4*>(Kloc + e + p0), k1);
    unpack8(*reinterpret_cast<const uint4*>(Kloc + e + 64 + p0), k2);
    rotate8(k1, k2, rope_offset + j, rr, p0);
    bf16x8_t h1, l1, h2, l2;
    split8(k1, h1, l1);
    split8(k2, h2, l2);
    kh1 = u4(h1); kl1 = u4(l1); kh2 = u4(h2); kl2 = u4(l2);
    v1 = *reinterpret_cast<const uint4*>(Vloc + e + p0);
    v2 = *reinterpret_cast<const uint4*>(Vloc + e + 64 + p0);
  }
  const int64_t row = (((int64_t)b * Hkv + g) * NK + kk) * D;
  *reinterpret_cast<uint4*>(Kh + row + p0) = kh1; *reinterpret_cast<uint4*>(Kh + row + 64 + p0) = kh2;
  *reinterpret_cast<uint4*>(Kl + row + p0) = kl1; *reinterpret_cast<uint4*>(Kl + row + 64 + p0) = kl2;
  *reinterpret_cast<uint4*>(Vc + row + p0) = v1; *reinterpret_cast<uint4*>(Vc + row + 64 + p0) = v2;
  *reinterpret_cast<uint4*>(&tile[0][r][p0]) = kh1; *reinterpret_cast<uint4*>(&tile[0][r][64 + p0]) = kh2;
  *reinterpret_cast<uint4*>(&tile[1][r][p0]) = kl1; *reinterpret_cast<uint4*>(&tile[1][r][64 + p0]) = kl2;
  if (M + kk < Mmax) {
    const int64_t z = (((int64_t)b * Mmax + M + kk) * Hkv + g) * D;
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      *reinterpret_cast<float4*>(dKmem + z + p0 + 4 * q) = zero;
      *reinterpret_cast<float4*>(dKmem + z + 64 + p0 + 4 * q) = zero;
      *reinterpret_cast<float4*>(dVmem + z + p0 + 4 * q) = zero;
      *reinterpret_cast<float4*>(dVmem + z + 64 + p0 + 4 * q) = zero;
    }
  }
  __syncthreads();
  uint16_t* const dst[2] = {KTh, KTl};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int id = tid + 256 * k;
    const int a = id >> 9, rb = (id >> 8) & 1, d = (id >> 1) & (D - 1), hf = id & 1;
    const int64_t blk = ((int64_t)b * Hkv + g) * (NK / 16) + kt * 2 + rb;
    *reinterpret_cast<uint4*>(dst[a] + (blk * D + d) * 16 + 8 * hf) = tile_blk8(tile[a], 16 * rb, hf, d);
  }
}

// Both preparations in one launch: workgroups [0, n_q) take query tiles (row tile,
// q-head, query), the rest key tiles (key tile, kv-head, query).
__global__ void __launch_bounds__(256)
bwd_prep_kernel(const PrepArgs A, const RopeRev rr) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[4][32][TS];      // Qh, Ql, Oh, Ol or Kh, Kl
  const int n_rt = A.Tq32 / 32, n_kt = A.NK / 32;
  const int64_t n_q = (int64_t)n_rt * A.Hq * A.B;
  int64_t id = blockIdx.x;
  if (id < n_q) {
    const int rt = (int)(id % n_rt), h = (int)(id / n_rt % A.Hq), b = (int)(id / ((int64_t)n_rt * A.Hq));
    prep_q_tile(A.Q, A.dO, A.Tq, A.Tq32, A.Hq, A.Tl, A.rope_offset, rr, A.Qh, A.Ql, A.QTh, A.QTl, A.Oh, A.Ol, A.OTh,
                A.OTl, rt, h, b, tile, A.O, A.lse, A.LSE2, A.DLT);
  } else {
    id -= n_q;
    const int kt = (int)(id % n_kt), g = (int)(id / n_kt % A.Hkv), b = (int)(id / ((int64_t)n_kt * A.Hkv));
    prep_k_tile(A.Kloc, A.Vloc, A.Tl, A.Hkv, A.Kmem, A.Vmem, A.mstride, A.Mmax, A.mem_len, A.NK, A.rope_offset, rr,
                A.Kh, A.Kl, A.KTh, A.KTl, A.Vc, A.dKmem, A.dVmem, kt, g, b, tile);
  }
}

struct Ops {
  const uint16_t *Qh, *Ql, *QTh, *QTl, *Oh, *Ol, *OTh, *OTl, *Kh, *Kl, *KTh, *KTl, *Vc;
};

// C-register layout of v_mfma_f32_32x32x16_bf16: register i of lane l holds
// row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32.  With A = keys x D and
// B = D x rows (S^T = K Q^T) a lane therefore holds one query row (column l % 32)
// and 16 of the tile's keys.

// One key tile's A operands for S^T = K Q^T and dP^T = V dO^T (this lane's key row),
// and the transposed keys that are the B operand of dQ += dS K.
struct KTile {
  bf16x8_t kh[8], kl[8], v[8];
};
struct KTTile {
  bf16x8_t h[2][4], l[2][4];
};
__device__ __forceinline__ void load_ktile(const Ops& op, int64_t kbase, int kt, int col, int hf, KTile& t) {
  const int64_t kr = (kbase + kt * 32 + col) * D + 8 * hf;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    t.kh[ks] = ld8(op.Kh + kr + 16 * ks);
    t.kl[ks] = ld8(op.Kl + kr + 16 * ks);
    t.v[ks] = ld8(op.Vc + kr + 16 * ks);
  }
}
__device__ __forceinline__ void load_kttile(const Ops& op, int64_t tbase, int NK, int kt, int col, int hf,
                                            KTTile& t) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int64_t a = ((tbase + kt * 2 + kb) * D + 32 * db + col) * 16 + 8 * hf;
      t.h[kb][db] = ld8(op.KTh + a);
      t.l[kb][db] = ld8(op.KTl + a);
    }
}

// Pass 1 (STATS) or pass 2 of the query side for rows [32 rt, 32 rt + 32) of q-head h.
// STATS: row max, sum of exponentials and sum of P * dP online over this wave's key
// tiles, merged over the waves into the row's log2-sum-exp and Delta.  Otherwise:
// dS^T per tile and dQ += dS K, merged, scaled and rotated back.
template <bool STATS>
__device__ __forceinline__ void dq_pass(const Ops& op, const int32_t* __restrict__ mem_len, int Tq, int Tq32, int Hq,
                                        int Tl, int Hkv, int Mmax, int NK, int rope_offset, const RopeRev& rr,
                                        float scale_log2e, float scale, float* __restrict__ LSE2,
                                        float* __restrict__ DLT, float* __restrict__ dQ, int rt, int h, int b,
                                        float (*part)[32][PSTRIDE], float (*stat)[32]) {
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, hf = lane >> 5;
  const int g = h / (Hq / Hkv);
  const int M = clamp_mem(mem_len, b, Mmax);
  const int r0 = rt * 32;
  const int last = r0 + 31 < Tq - 1 ? r0 + 31 : Tq - 1;
  const int n_kt = (M + (Tl - Tq) + last + 1 + 31) / 32;   // tiles up to the last row's causal limit
  const int row = r0 + col;                                // this lane's query row
  const int climit = (Tl - Tq) + row;                      // local keys j <= climit are visible

  // resident B operands: the rotated query row and its dO row, split
  const int64_t qrow = (((int64_t)b * Hq + h) * Tq32 + row) * D + 8 * hf;
  bf16x8_t bqh[8], bql[8], boh[8], bol[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    bqh[ks] = ld8(op.Qh + qrow + 16 * ks);
    bql[ks] = ld8(op.Ql + qrow + 16 * ks);
    boh[ks] = ld8(op.Oh + qrow + 16 * ks);
    bol[ks] = ld8(op.Ol + qrow + 16 * ks);
  }
  const int64_t kbase = ((int64_t)b * Hkv + g) * NK;

  // S^T and dP^T of a loaded key tile (raw products; scores still unscaled)
  auto tile_products = [&](const KTile& t, f32x16_t& s, f32x16_t& dp) {
    s = (f32x16_t){};
    dp = (f32x16_t){};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s = mfma(t.kh[ks], bqh[ks], s);
      s = mfma(t.kh[ks], bql[ks], s);
      s = mfma(t.kl[ks], bqh[ks], s);
      dp = mfma(t.v[ks], boh[ks], dp);
      dp = mfma(t.v[ks], bol[ks], dp);
    }
  };
  // the wave's key tiles kt = wave, wave + NW, ...: each tile's rows are loaded one
  // tile ahead, so their memory latency overlaps the previous tile's products
  KTile cur, nxt;
  if (wave < n_kt) load_ktile(op, kbase, wave, col, hf, cur);
  auto visible = [&](int key) { return key < M || (key - M < Tl && key - M <= climit); };

  if constexpr (STATS) {
  // ---- pass 1: row max (log2 domain), sum of exponentials and sum of P * dP, online
  float m = -INFINITY, l = 0.f, a = 0.f;
  for (int kt = wave; kt < n_kt; kt += NW) {
    if (kt + NW < n_kt) load_ktile(op, kbase, kt + NW, col, hf, nxt);
    f32x16_t s, dp;
    tile_products(cur, s, dp);
    float x[16];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kt * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
      x[i] = visible(key) ? s[i] * scale_log2e : -INFINITY;
      mx = fmaxf(mx, x[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    if (mn != -INFINITY) {
      float ls = 0.f, as = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = exp2f(x[i] - mn);
        ls += e;
        as += e * dp[i];
      }
      ls += __shfl_xor(ls, 32);
      as += __shfl_xor(as, 32);
      const float sc = exp2f(m - mn);        // 0 while m is still -inf
      l = l * sc + ls;
      a = a * sc + as;
      m = mn;
    }
    cur = nxt;
  }
  if (hf == 0) { stat[wave][col] = m; stat[NW + wave][col] = l; stat[2 * NW + wave][col] = a; }
  __syncthreads();
  if (tid < 32) {
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, stat[w][tid]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (stat[w][tid] != -INFINITY) {
        const float sc = exp2f(stat[w][tid] - mm);
        L += stat[NW + w][tid] * sc;
        A += stat[2 * NW + w][tid] * sc;
      }
    }
    const bool valid = r0 + tid < Tq;
    LSE2[((int64_t)b * Hq + h) * Tq32 + r0 + tid] = valid ? mm + log2f(L) : INFINITY;   // padded rows: P = 0
    DLT[((int64_t)b * Hq + h) * Tq32 + r0 + tid] = valid ? A / L : 0.f;
  }
  } else {
  // ---- pass 2: dS^T per tile, dQ[row][dim] += dS K (contraction over the tile's keys)
  const float lse_r = LSE2[((int64_t)b * Hq + h) * Tq32 + row];
  const float dlt_r = DLT[((int64_t)b * Hq + h) * Tq32 + row];
  f32x16_t acc[4] = {};
  const int64_t tbase = ((int64_t)b * Hkv + g) * (NK / 16);             // first 16-key block of the head
  for (int kt = wave; kt < n_kt; kt += NW) {
    if (kt + NW < n_kt) load_ktile(op, kbase, kt + NW, col, hf, nxt);
    KTTile kt_t;
    load_kttile(op, tbase, NK, kt, col, hf, kt_t);
    f32x16_t s, dp;
    tile_products(cur, s, dp);
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kt * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
      const float p = visible(key) ? exp2f(s[i] * scale_log2e - lse_r) : 0.f;
      ds[i] = p * (dp[i] - dlt_r);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8_t ah, al;
      split8(ds + 8 * kb, ah, al);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        acc[db] = mfma(ah, kt_t.h[kb][db], acc[db]);
        acc[db] = mfma(ah, kt_t.l[kb][db], acc[db]);
        acc[db] = mfma(al, kt_t.h[kb][db], acc[db]);
      }
    }
    cur = nxt;
  }
  // acc[db] register i: row 8 (i / 4) + 4 hf + i % 4, dim 32 db + col
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) part[wave][8 * (i / 4) + 4 * hf + (i % 4)][32 * db + col] = acc[db][i];
  __syncthreads();
  // waves added in order, scaled, rotated back by the row's position
  for (int e = tid; e < 32 * (D / 2); e += THREADS) {
    const int r = e / (D / 2), pr = e % (D / 2);
    if (r0 + r >= Tq) continue;
    float g1 = 0.f, g2 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) { g1 += part[w][r][pr]; g2 += part[w][r][pr + 64]; }
    g1 *= scale;
    g2 *= scale;
    float c, s;
    rope_cs(rope_offset + (Tl - Tq) + r0 + r, rr.rev[pr], &c, &s);
    float* o = dQ + (((int64_t)b * Tq + r0 + r) * Hq + h) * D;
    o[pr] = g1 * c + g2 * s;
    o[pr + 64] = g2 * c - g1 * s;
  }
  }
}

__global__ void __launch_bounds__(THREADS, 1)
bwd_stats_kernel(const Ops op, const int32_t* __restrict__ mem_len, int Tq, int Tq32, int Hq, int Tl, int Hkv, int Mmax,
                 int NK, int rope_offset, const RopeRev rr, float scale_log2e, float* __restrict__ LSE2,
                 float* __restrict__ DLT) {
  __shared__ float stat[3 * NW][32];
  dq_pass<true>(op, mem_len, Tq, Tq32, Hq, Tl, Hkv, Mmax, NK, rope_offset, rr, scale_log2e, 0.f, LSE2, DLT, nullptr,
                blockIdx.x, blockIdx.y, blockIdx.z, nullptr, stat);
}

// C layout with A = rows x D and B = D x keys (S = Q K^T): a lane holds one key
// (column l % 32) and 16 of the tile's rows.
// Key side for key tile kt of q-heads hp*hpw .. hp*hpw + hpw - 1: their (unscaled,
// rotated-frame) share of dK and dV for the tile's 32 keys, written to
// dKp / dVp [B, Hq / hpw, NK, D]; the waves take the (head, row tile) pairs that can
// see the tile.
__device__ __forceinline__ void dkv_body(const Ops& op, const int32_t* __restrict__ mem_len, int Tq, int Tq32, int Hq,
                                         int Tl, int Hkv, int Mmax, int NK, float scale_log2e,
                                         const float* __restrict__ LSE2, const float* __restrict__ DLT,
                                         float* __restrict__ dKp, float* __restrict__ dVp, int kt, int hp, int hpw,
                                         int b, float (*part)[32][PSTRIDE]) {
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, hf = lane >> 5;
  const int M = clamp_mem(mem_len, b, Mmax);
  const int nkb = M + Tl;
  const int k0 = kt * 32;
  if (k0 >= nkb) return;
  const int g = hp * hpw / (Hq / Hkv);
  // row tiles that see any key of this tile: all of them if it holds a memory key
  int rt_lo = 0;
  if (k0 >= M) {
    const int i0 = (k0 - M) - (Tl - Tq);
    rt_lo = i0 > 0 ? i0 / 32 : 0;
  }
  const int n_rt = Tq32 / 32;
  const int n_items = hpw * (n_rt - rt_lo);
  const int key = k0 + col;                       // this lane's key
  const bool kvalid = key < nkb;
  const int kloc = key - M;                       // local index when key >= M

  // resident B operands: this lane's key row (split) and value row
  const int64_t kr = (((int64_t)b * Hkv + g) * NK + key) * D + 8 * hf;
  bf16x8_t bkh[8], bkl[8], bv[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    bkh[ks] = ld8(op.Kh + kr + 16 * ks);
    bkl[ks] = ld8(op.Kl + kr + 16 * ks);
    bv[ks] = ld8(op.Vc + kr + 16 * ks);
  }
  f32x16_t dk[4] = {}, dv[4] = {};
  for (int it = wave; it < n_items; it += NW) {
    const int h = hp * hpw + it % hpw;
    const int rb = (rt_lo + it / hpw) * 32;
    const int64_t hq = ((int64_t)b * Hq + h) * Tq32;
    const int64_t qr = (hq + rb + col) * D + 8 * hf;
    // every operand load of the item is issued before the first product: one
    // memory latency per item instead of one per k-step
    bf16x8_t aqh[8], aql[8], aoh[8], aol[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      aqh[ks] = ld8(op.Qh + qr + 16 * ks);
      aql[ks] = ld8(op.Ql + qr + 16 * ks);
      aoh[ks] = ld8(op.Oh + qr + 16 * ks);
      aol[ks] = ld8(op.Ol + qr + 16 * ks);
    }
    float4 L4s[4], D4s[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      L4s[q] = *reinterpret_cast<const float4*>(LSE2 + hq + rb + 8 * q + 4 * hf);
      D4s[q] = *reinterpret_cast<const float4*>(DLT + hq + rb + 8 * q + 4 * hf);
    }
    const int64_t tq = ((int64_t)b * Hq + h) * (Tq32 / 16) + rb / 16;     // first 16-row block of the tile
    bf16x8_t toh[2][4], tol[2][4], tqh[2][4], tql[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int64_t t = ((tq + kb) * D + 32 * db + col) * 16 + 8 * hf;
        toh[kb][db] = ld8(op.OTh + t);
        tol[kb][db] = ld8(op.OTl + t);
        tqh[kb][db] = ld8(op.QTh + t);
        tql[kb][db] = ld8(op.QTl + t);
      }
    f32x16_t s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s = mfma(aqh[ks], bkh[ks], s);
      s = mfma(aql[ks], bkh[ks], s);
      s = mfma(aqh[ks], bkl[ks], s);
      dp = mfma(aoh[ks], bv[ks], dp);
      dp = mfma(aol[ks], bv[ks], dp);
    }
    // register i: row rb + 8 (i / 4) + 4 hf + i % 4 of this lane's key
    float p[16], ds[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 L4 = L4s[q];
      const float4 D4 = D4s[q];
      const float Lv[4] = {L4.x, L4.y, L4.z, L4.w}, Dv[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * q + e;
        const int r = rb + 8 * q + 4 * hf + e;
        const bool vis = kvalid && (key < M || kloc <= (Tl - Tq) + r);
        p[i] = vis ? exp2f(s[i] * scale_log2e - Lv[e]) : 0.f;
        ds[i] = p[i] * (dp[i] - Dv[e]);
      }
    }
    // dV[key][dim] += P^T dO and dK[key][dim] += dS^T Qrot, contraction over the tile's rows
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8_t ph, pl, sh, sl;
      split8(p + 8 * kb, ph, pl);
      split8(ds + 8 * kb, sh, sl);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8_t oh = toh[kb][db], ol = tol[kb][db], qh = tqh[kb][db], ql = tql[kb][db];
        dv[db] = mfma(ph, oh, dv[db]);
        dv[db] = mfma(ph, ol, dv[db]);
        dv[db] = mfma(pl, oh, dv[db]);
        dk[db] = mfma(sh, qh, dk[db]);
        dk[db] = mfma(sh, ql, dk[db]);
        dk[db] = mfma(sl, qh, dk[db]);
      }
    }
  }

  // ---- merge the waves in order; dv/dk register i: key 8 (i / 4) + 4 hf + i % 4, dim 32 db + col
  for (int pass = 0; pass < 2; ++pass) {
    if (pass) __syncthreads();                  // the previous pass has read the merge area
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        part[wave][8 * (i / 4) + 4 * hf + (i % 4)][32 * db + col] = pass ? dk[db][i] : dv[db][i];
    __syncthreads();
    float* dst = (pass ? dKp : dVp) + (((int64_t)b * (Hq / hpw) + hp) * NK + k0) * D;
    for (int e = tid; e < 32 * (D / 4); e += THREADS) {
      const int kk = e / (D / 4), d4 = 4 * (e % (D / 4));
      float4 v = *reinterpret_cast<const float4*>(&part[0][kk][d4]);
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const float4 x = *reinterpret_cast<const float4*>(&part[w][kk][d4]);
        v.x += x.x; v.y += x.y; v.z += x.z; v.w += x.w;
      }
      *reinterpret_cast<float4*>(dst + kk * D + d4) = v;
    }
  }
}

// dK and dV of key tile kt of kv-head g: its q-heads' shares added in head order,
// dK scaled and (local keys) rotated back by the key's position.  One thread per
// (key, four rotation pairs): every load is issued before any sum is needed.
__global__ void __launch_bounds__(512)
bwd_kv_reduce_kernel(const int32_t* __restrict__ mem_len, int Hq, int Tl, int Hkv, int Mmax, int NK, int rope_offset,
                     const RopeRev rr, float scale, const float* __restrict__ dKp, const float* __restrict__ dVp,
                     float* __restrict__ dKloc, float* __restrict__ dVloc, float* __restrict__ dKmem,
                     float* __restrict__ dVmem) {
  constexpr int GMAX = 4;                       // q-heads per kv-head with all loads in flight at once
  const int kt = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int M = clamp_mem(mem_len, b, Mmax);
  const int hpw = KV_HPW;   // q-heads per partial (as in the key side)
  const int G = Hq / Hkv / hpw, NP = Hq / hpw;
  const int kk = tid >> 4, p4 = 4 * (tid & 15);  // key in the tile, first of four pairs
  const int kg = kt * 32 + kk;
  if (kg >= M + Tl) return;
  float4 k1 = make_float4(0.f, 0.f, 0.f, 0.f), k2 = k1, v1 = k1, v2 = k1;
  for (int j0 = 0; j0 < G; j0 += GMAX) {
    float4 a[GMAX], c[GMAX], e[GMAX], f[GMAX];
#pragma unroll
    for (int j = 0; j < GMAX; ++j) {
      if (j0 + j < G) {
        const int64_t r = (((int64_t)b * NP + g * G + j0 + j) * NK + kg) * D + p4;
        a[j] = *reinterpret_cast<const float4*>(dKp + r);
        c[j] = *reinterpret_cast<const float4*>(dKp + r + 64);
        e[j] = *reinterpret_cast<const float4*>(dVp + r);
        f[j] = *reinterpret_cast<const float4*>(dVp + r + 64);
      }
    }
#pragma unroll
    for (int j = 0; j < GMAX; ++j) {
      if (j0 + j < G) {
        k1.x += a[j].x; k1.y += a[j].y; k1.z += a[j].z; k1.w += a[j].w;
        k2.x += c[j].x; k2.y += c[j].y; k2.z += c[j].z; k2.w += c[j].w;
        v1.x += e[j].x; v1.y += e[j].y; v1.z += e[j].z; v1.w += e[j].w;
        v2.x += f[j].x; v2.y += f[j].y; v2.z += f[j].z; v2.w += f[j].w;
      }
    }
  }
  float x1[4] = {k1.x * scale, k1.y * scale, k1.z * scale, k1.w * scale};
  float x2[4] = {k2.x * scale, k2.y * scale, k2.z * scale, k2.w * scale};
  float *ok, *ov;
  if (kg < M) {
    ok = dKmem + (((int64_t)b * Mmax + kg) * Hkv + g) * D;
    ov = dVmem + (((int64_t)b * Mmax + kg) * Hkv + g) * D;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float cs, sn;
      rope_cs(rope_offset + (kg - M), rr.rev[p4 + q], &cs, &sn);
      const float y1 = x1[q] * cs + x2[q] * sn, y2 = x2[q] * cs - x1[q] * sn;
      x1[q] = y1;
      x2[q] = y2;
    }
    ok = dKloc + (((int64_t)b * Tl + kg - M) * Hkv + g) * D;
    ov = dVloc + (((int64_t)b * Tl + kg - M) * Hkv + g) * D;
  }
  *reinterpret_cast<float4*>(ok + p4) = make_float4(x1[0], x1[1], x1[2], x1[3]);
  *reinterpret_cast<float4*>(ok + p4 + 64) = make_float4(x2[0], x2[1], x2[2], x2[3]);
  *reinterpret_cast<float4*>(ov + p4) = v1;
  *reinterpret_cast<float4*>(ov + p4 + 64) = v2;
}

// The query-side gradient (workgroups [0, n_dq): row tile, q-head, query) and the
// key side (the rest: key tile, pair of q-heads, query) in one launch, so the two kinds run
// side by side on different CUs.
__global__ void __launch_bounds__(THREADS, 1)
bwd_grad_kernel(const Ops op, const int32_t* __restrict__ mem_len, int B, int Tq, int Tq32, int Hq, int Tl, int Hkv,
                int Mmax, int NK, int rope_offset, const RopeRev rr, float scale_log2e, float scale,
                float* __restrict__ LSE2, float* __restrict__ DLT, float* __restrict__ dQ, float* __restrict__ dKp,
                float* __restrict__ dVp) {
  __shared__ __attribute__((aligned(16))) float part[NW][32][PSTRIDE];
  const int n_rt = Tq32 / 32, n_kt = NK / 32;
  const int64_t n_dq = (int64_t)n_rt * Hq * B;
  int64_t id = blockIdx.x;
  if (id < n_dq) {
    const int rt = (int)(id % n_rt), h = (int)(id / n_rt % Hq), b = (int)(id / ((int64_t)n_rt * Hq));
    dq_pass<false>(op, mem_len, Tq, Tq32, Hq, Tl, Hkv, Mmax, NK, rope_offset, rr, scale_log2e, scale, LSE2, DLT, dQ,
                   rt, h, b, part, nullptr);
  } else {
    id -= n_dq;
    const int hpw = KV_HPW, n_hp = Hq / hpw;
    const int kt = (int)(id % n_kt), hp = (int)(id / n_kt % n_hp), b = (int)(id / ((int64_t)n_kt * n_hp));
    dkv_body(op, mem_len, Tq, Tq32, Hq, Tl, Hkv, Mmax, NK, scale_log2e, LSE2, DLT, dKp, dVp, kt, hp, hpw, b, part);
  }
}

struct BwdLayout {
  int Tq32, NK;
  size_t q[8], k[5], lse, dlt, kp, vp, total;
};

BwdLayout layout(int B, int Tq, int Hq, int Tl, int Hkv, int Mmax) {
  BwdLayout L;
  L.Tq32 = (Tq + 31) / 32 * 32;
  L.NK = (Mmax + Tl + 31) / 32 * 32;
  size_t o = 0;
  auto take = [&o](size_t bytes) {
    const size_t at = o;
    o += (bytes + 255) & ~(size_t)255;
    return at;
  };
  const size_t qsz = (size_t)B * Hq * L.Tq32 * D * 2, ksz = (size_t)B * Hkv * L.NK * D * 2;
  for (int i = 0; i < 8; ++i) L.q[i] = take(qsz);
  for (int i = 0; i < 5; ++i) L.k[i] = take(ksz);
  L.lse = take((size_t)B * Hq * L.Tq32 * 4);
  L.dlt = take((size_t)B * Hq * L.Tq32 * 4);
  L.kp = take((size_t)B * Hq * L.NK * D * 4);
  L.vp = take((size_t)B * Hq * L.NK * D * 4);
  L.total = o;
  return L;
}

}  // namespace

size_t attn_bwd_workspace(int B, int Tq, int Hq, int Tl, int Hkv, int Mmax) {
  return layout(B, Tq, Hq, Tl, Hkv, Mmax).total;
}

int launch_attn_bwd(const uint16_t* Q, int B, int Tq, int Hq, const uint16_t* Kloc, const uint16_t* Vloc, int Tl,
                    int Hkv, const uint16_t* Kmem, const uint16_t* Vmem, int64_t mem_entry_stride, int Mmax,
                    const int32_t* mem_len, int rope_offset, double rope_base, float scale, const float* dO,
                    const float* O, const float* lse_saved, float* dQ, float* dKloc, float* dVloc, float* dKmem,
                    float* dVmem, void* workspace, hipStream_t stream) {
  const BwdLayout L = layout(B, Tq, Hq, Tl, Hkv, Mmax);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  uint16_t* qa[8];
  uint16_t* ka[5];
  for (int i = 0; i < 8; ++i) qa[i] = reinterpret_cast<uint16_t*>(ws + L.q[i]);
  for (int i = 0; i < 5; ++i) ka[i] = reinterpret_cast<uint16_t*>(ws + L.k[i]);
  float* lse = reinterpret_cast<float*>(ws + L.lse);
  float* dlt = reinterpret_cast<float*>(ws + L.dlt);
  float* kp = reinterpret_cast<float*>(ws + L.kp);
  float* vp = reinterpret_cast<float*>(ws + L.vp);
  RopeRev rr;
  const double two_pi = 6.283185307179586;
  for (int i = 0; i < D / 2; ++i) rr.rev[i] = pow(rope_base, -2.0 * i / D) / two_pi;
  const float scale_log2e = scale * 1.4426950408889634f;

  const bool saved = O && lse_saved;
  const PrepArgs pa{Q, Kloc, Vloc, Kmem, Vmem, dO, saved ? O : nullptr, lse_saved, lse, dlt, mem_len, B, Tq, L.Tq32,
                    Hq, Tl, Hkv, Mmax, L.NK, rope_offset,
                    mem_entry_stride, qa[0], qa[1], qa[2], qa[3], qa[4], qa[5], qa[6], qa[7], ka[0], ka[1], ka[2],
                    ka[3], ka[4], dKmem, dVmem};
  const int64_t n_prep = (int64_t)(L.Tq32 / 32) * Hq * B + (int64_t)(L.NK / 32) * Hkv * B;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)n_prep), dim3(256), 0, stream, pa, rr);
  MSA_CHECK_LAUNCH();
  const Ops op{qa[0], qa[1], qa[2], qa[3], qa[4], qa[5], qa[6], qa[7], ka[0], ka[1], ka[2], ka[3], ka[4]};
  if (!saved) {
    hipLaunchKernelGGL(bwd_stats_kernel, dim3((unsigned)(L.Tq32 / 32), (unsigned)Hq, (unsigned)B), dim3(THREADS), 0,
                       stream, op, mem_len, Tq, L.Tq32, Hq, Tl, Hkv, Mmax, L.NK, rope_offset, rr, scale_log2e, lse, dlt);
    MSA_CHECK_LAUNCH();
  }
  const int hpw = KV_HPW;
  const int64_t n_wg = (int64_t)(L.Tq32 / 32) * Hq * B + (int64_t)(L.NK / 32) * (Hq / hpw) * B;
  hipLaunchKernelGGL(bwd_grad_kernel, dim3((unsigned)n_wg), dim3(THREADS), 0, stream, op, mem_len, B, Tq, L.Tq32, Hq,
                     Tl, Hkv, Mmax, L.NK, rope_offset, rr, scale_log2e, scale, lse, dlt, dQ, kp, vp);
  MSA_CHECK_LAUNCH();
  hipLaunchKernelGGL(bwd_kv_reduce_kernel, dim3((unsigned)(L.NK / 32), (unsigned)Hkv, (unsigned)B), dim3(512), 0,
                     stream, mem_len, Hq, Tl, Hkv, Mmax, L.NK, rope_offset, rr, scale, kp, vp, dKloc, dVloc, dKmem,
                     dVmem);
  MSA_CHECK_LAUNCH();

  return MSA_OK;
}

}  // namespace msa
