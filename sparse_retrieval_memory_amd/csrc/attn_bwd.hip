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
//   bwd_prep_q / bwd_prep_k   rotate Q and the local keys, split every fp32
//       operand into bf16 hi + lo parts (x = hi + lo, |lo| <= 2^-9 |x|) and lay
//       the operands out per head, row-major and transposed, padded to 32-row /
//       32-key tiles with zeros; keys in the forward's order (memory, then local)
//   bwd_dq_kernel   32 query rows of one q-head per workgroup; the 4 waves take
//       every 4th key tile.  Pass 1: row max, sum and Delta online (S^T = K Q^T
//       and dP^T = V dO^T on v_mfma_f32_32x32x16_bf16, one query row per lane
//       pair), merged over the waves -> log2-sum-exp and Delta per row.  Pass 2:
//       dS^T per tile and dQ += dS K with the key dimension as the contraction.
//   bwd_dkv_kernel  32 keys of one kv-head per workgroup, the K and V rows
//       resident as B operands; the waves split the (q-head, row tile) pairs;
//       S = Q K^T and dP = dO V^T give P and dS with one key per lane pair, then
//       dV += P^T dO and dK += dS^T Qrot with the row dimension as the
//       contraction (transposed dO and Qrot from the prep kernels).
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
// B operand of a product whose contraction runs over rows / keys: 8 values of a
// transposed row at k = base + {0..3} and base + 8 + {0..3} (the order in which a
// lane holds the rows of an MFMA result, see the C-register layout below)
__device__ __forceinline__ bf16x8_t ld_perm(const uint16_t* p) {
  const uint2 a = *reinterpret_cast<const uint2*>(p), b = *reinterpret_cast<const uint2*>(p + 8);
  return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int clamp_mem(const int32_t* mem_len, int b, int Mmax) {
  int M = mem_len[b];
  return M < 0 ? 0 : (M > Mmax ? Mmax : M);
}

// Q rows: rotated at rope_offset + (Tl - Tq) + i and split; dO rows split.  Row-major
// [B, Hq, Tq32, D] and transposed [B, Hq, D, Tq32]; rows >= Tq are zeros.
__global__ void __launch_bounds__(64)
bwd_prep_q_kernel(const uint16_t* __restrict__ Q, const float* __restrict__ dO, int Tq, int Tq32, int Hq, int Tl,
                  int rope_offset, const RopeRev rr, uint16_t* __restrict__ Qh, uint16_t* __restrict__ Ql,
                  uint16_t* __restrict__ QTh, uint16_t* __restrict__ QTl, uint16_t* __restrict__ Oh,
                  uint16_t* __restrict__ Ol, uint16_t* __restrict__ OTh, uint16_t* __restrict__ OTl) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, p = threadIdx.x;
  float x[4] = {0.f, 0.f, 0.f, 0.f};       // q(p), q(p + 64), dO(p), dO(p + 64)
  if (i < Tq) {
    const int64_t src = (((int64_t)b * Tq + i) * Hq + h) * D;
    const float q1 = bits_f32(Q[src + p]), q2 = bits_f32(Q[src + p + 64]);
    float c, s;
    rope_cs(rope_offset + (Tl - Tq) + i, rr.rev[p], &c, &s);
    x[0] = q1 * c - q2 * s;
    x[1] = q2 * c + q1 * s;
    x[2] = dO[src + p];
    x[3] = dO[src + p + 64];
  }
  uint16_t hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = bf16_bits(x[e]);
    lo[e] = bf16_bits(x[e] - bits_f32(hi[e]));
  }
  const int64_t row = (((int64_t)b * Hq + h) * Tq32 + i) * D;
  Qh[row + p] = hi[0]; Qh[row + p + 64] = hi[1]; Ql[row + p] = lo[0]; Ql[row + p + 64] = lo[1];
  Oh[row + p] = hi[2]; Oh[row + p + 64] = hi[3]; Ol[row + p] = lo[2]; Ol[row + p + 64] = lo[3];
  const int64_t c0 = (((int64_t)b * Hq + h) * D + p) * Tq32 + i, c1 = c0 + (int64_t)64 * Tq32;
  QTh[c0] = hi[0]; QTh[c1] = hi[1]; QTl[c0] = lo[0]; QTl[c1] = lo[1];
  OTh[c0] = hi[2]; OTh[c1] = hi[3]; OTl[c0] = lo[2]; OTl[c1] = lo[3];
}

// Keys in the forward's order (memory entries, then local keys rotated at rope_offset + j),
// split, row-major [B, Hkv, NK, D] and transposed [B, Hkv, D, NK]; V row-major (exact bf16).
// Keys >= M + Tl are zeros.  Also zeroes the memory-gradient entries [M, Mmax).
__global__ void __launch_bounds__(64)
bwd_prep_k_kernel(const uint16_t* __restrict__ Kloc, const uint16_t* __restrict__ Vloc, int Tl, int Hkv,
                  const uint16_t* __restrict__ Kmem, const uint16_t* __restrict__ Vmem, int64_t mstride, int Mmax,
                  const int32_t* __restrict__ mem_len, int NK, int rope_offset, const RopeRev rr,
                  uint16_t* __restrict__ Kh, uint16_t* __restrict__ Kl, uint16_t* __restrict__ KTh,
                  uint16_t* __restrict__ KTl, uint16_t* __restrict__ Vc, float* __restrict__ dKmem,
                  float* __restrict__ dVmem) {
  const int kk = blockIdx.x, g = blockIdx.y, b = blockIdx.z, p = threadIdx.x;
  const int M = clamp_mem(mem_len, b, Mmax);
  uint16_t kh[2] = {0, 0}, kl[2] = {0, 0}, v[2] = {0, 0};
  if (kk < M) {
    const int64_t e = ((int64_t)b * Mmax + kk) * mstride + (int64_t)g * D;
    kh[0] = Kmem[e + p]; kh[1] = Kmem[e + p + 64];
    v[0] = Vmem[e + p]; v[1] = Vmem[e + p + 64];
  } else if (kk < M + Tl) {
    const int j = kk - M;
    const int64_t e = (((int64_t)b * Tl + j) * Hkv + g) * D;
    const float k1 = bits_f32(Kloc[e + p]), k2 = bits_f32(Kloc[e + p + 64]);
    float c, s;
    rope_cs(rope_offset + j, rr.rev[p], &c, &s);
    const float y[2] = {k1 * c - k2 * s, k2 * c + k1 * s};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      kh[t] = bf16_bits(y[t]);
      kl[t] = bf16_bits(y[t] - bits_f32(kh[t]));
    }
    v[0] = Vloc[e + p]; v[1] = Vloc[e + p + 64];
  }
  const int64_t row = (((int64_t)b * Hkv + g) * NK + kk) * D;
  Kh[row + p] = kh[0]; Kh[row + p + 64] = kh[1]; Kl[row + p] = kl[0]; Kl[row + p + 64] = kl[1];
  Vc[row + p] = v[0]; Vc[row + p + 64] = v[1];
  const int64_t c0 = (((int64_t)b * Hkv + g) * D + p) * NK + kk, c1 = c0 + (int64_t)64 * NK;
  KTh[c0] = kh[0]; KTh[c1] = kh[1]; KTl[c0] = kl[0]; KTl[c1] = kl[1];
  if (M + kk < Mmax) {
    const int64_t z = (((int64_t)b * Mmax + M + kk) * Hkv + g) * D;
    dKmem[z + p] = 0.f; dKmem[z + p + 64] = 0.f;
    dVmem[z + p] = 0.f; dVmem[z + p + 64] = 0.f;
  }
}

struct Ops {
  const uint16_t *Qh, *Ql, *QTh, *QTl, *Oh, *Ol, *OTh, *OTl, *Kh, *Kl, *KTh, *KTl, *Vc;
};

// C-register layout of v_mfma_f32_32x32x16_bf16: register i of lane l holds
// row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32.  With A = keys x D and
// B = D x rows (S^T = K Q^T) a lane therefore holds one query row (column l % 32)
// and 16 of the tile's keys.

__global__ void __launch_bounds__(THREADS, 1)
bwd_dq_kernel(const Ops op, const int32_t* __restrict__ mem_len, int Tq, int Tq32, int Hq, int Tl, int Hkv, int Mmax,
              int NK, int rope_offset, const RopeRev rr, float scale_log2e, float scale, float* __restrict__ LSE2,
              float* __restrict__ DLT, float* __restrict__ dQ) {
  __shared__ float m_sh[NW][32], l_sh[NW][32], a_sh[NW][32];
  __shared__ float lse_s[32], dlt_s[32];
  __shared__ __attribute__((aligned(16))) float part[NW][32][PSTRIDE];
  const int rt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
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

  // S^T and dP^T of key tile kt (raw products; scores still unscaled)
  auto tile_products = [&](int kt, f32x16_t& s, f32x16_t& dp) {
    const int64_t kr = (kbase + kt * 32 + col) * D + 8 * hf;
    s = (f32x16_t){};
    dp = (f32x16_t){};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t kh = ld8(op.Kh + kr + 16 * ks), kl = ld8(op.Kl + kr + 16 * ks), v = ld8(op.Vc + kr + 16 * ks);
      s = mfma(kh, bqh[ks], s);
      s = mfma(kh, bql[ks], s);
      s = mfma(kl, bqh[ks], s);
      dp = mfma(v, boh[ks], dp);
      dp = mfma(v, bol[ks], dp);
    }
  };
  auto visible = [&](int key) { return key < M || (key - M < Tl && key - M <= climit); };

  // ---- pass 1: row max (log2 domain), sum of exponentials and sum of P * dP, online
  float m = -INFINITY, l = 0.f, a = 0.f;
  for (int kt = wave; kt < n_kt; kt += NW) {
    f32x16_t s, dp;
    tile_products(kt, s, dp);
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
  }
  if (hf == 0) { m_sh[wave][col] = m; l_sh[wave][col] = l; a_sh[wave][col] = a; }
  __syncthreads();
  if (tid < 32) {
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, m_sh[w][tid]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (m_sh[w][tid] != -INFINITY) {
        const float sc = exp2f(m_sh[w][tid] - mm);
        L += l_sh[w][tid] * sc;
        A += a_sh[w][tid] * sc;
      }
    }
    const bool valid = r0 + tid < Tq;
    const float lse = valid ? mm + log2f(L) : INFINITY;   // padded rows: P = 0
    const float dl = valid ? A / L : 0.f;
    lse_s[tid] = lse;
    dlt_s[tid] = dl;
    LSE2[((int64_t)b * Hq + h) * Tq32 + r0 + tid] = lse;
    DLT[((int64_t)b * Hq + h) * Tq32 + r0 + tid] = dl;
  }
  __syncthreads();

  // ---- pass 2: dS^T per tile, dQ[row][dim] += dS K (contraction over the tile's keys)
  const float lse_r = lse_s[col], dlt_r = dlt_s[col];
  f32x16_t acc[4] = {};
  const int64_t tbase = ((int64_t)b * Hkv + g) * D;
  for (int kt = wave; kt < n_kt; kt += NW) {
    f32x16_t s, dp;
    tile_products(kt, s, dp);
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
      const int k0 = kt * 32 + 16 * kb + 4 * hf;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int64_t t = (tbase + 32 * db + col) * NK + k0;
        const bf16x8_t bh = ld_perm(op.KTh + t), bl = ld_perm(op.KTl + t);
        acc[db] = mfma(ah, bh, acc[db]);
        acc[db] = mfma(ah, bl, acc[db]);
        acc[db] = mfma(al, bh, acc[db]);
      }
    }
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

// C layout with A = rows x D and B = D x keys (S = Q K^T): a lane holds one key
// (column l % 32) and 16 of the tile's rows.
__global__ void __launch_bounds__(THREADS, 1)
bwd_dkv_kernel(const Ops op, const int32_t* __restrict__ mem_len, int Tq, int Tq32, int Hq, int Tl, int Hkv, int Mmax,
               int NK, int rope_offset, const RopeRev rr, float scale_log2e, float scale,
               const float* __restrict__ LSE2, const float* __restrict__ DLT, float* __restrict__ dKloc,
               float* __restrict__ dVloc, float* __restrict__ dKmem, float* __restrict__ dVmem) {
  __shared__ __attribute__((aligned(16))) float part[NW][32][PSTRIDE];
  const int kt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, hf = lane >> 5;
  const int M = clamp_mem(mem_len, b, Mmax);
  const int nkb = M + Tl;
  const int k0 = kt * 32;
  if (k0 >= nkb) return;
  const int G = Hq / Hkv;
  // row tiles that see any key of this tile: all of them if it holds a memory key
  int rt_lo = 0;
  if (k0 >= M) {
    const int i0 = (k0 - M) - (Tl - Tq);
    rt_lo = i0 > 0 ? i0 / 32 : 0;
  }
  const int n_rt = Tq32 / 32;
  const int n_items = G * (n_rt - rt_lo);
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
    const int h = g * G + it % G;
    const int rb = (rt_lo + it / G) * 32;
    const int64_t hq = ((int64_t)b * Hq + h) * Tq32;
    const int64_t qr = (hq + rb + col) * D + 8 * hf;
    f32x16_t s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t qh = ld8(op.Qh + qr + 16 * ks), ql = ld8(op.Ql + qr + 16 * ks);
      const bf16x8_t oh = ld8(op.Oh + qr + 16 * ks), ol = ld8(op.Ol + qr + 16 * ks);
      s = mfma(qh, bkh[ks], s);
      s = mfma(ql, bkh[ks], s);
      s = mfma(qh, bkl[ks], s);
      dp = mfma(oh, bv[ks], dp);
      dp = mfma(ol, bv[ks], dp);
    }
    // register i: row rb + 8 (i / 4) + 4 hf + i % 4 of this lane's key
    float p[16], ds[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 L4 = *reinterpret_cast<const float4*>(LSE2 + hq + rb + 8 * q + 4 * hf);
      const float4 D4 = *reinterpret_cast<const float4*>(DLT + hq + rb + 8 * q + 4 * hf);
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
    const int64_t tq = (((int64_t)b * Hq + h) * D) * Tq32;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8_t ph, pl, sh, sl;
      split8(p + 8 * kb, ph, pl);
      split8(ds + 8 * kb, sh, sl);
      const int r0 = rb + 16 * kb + 4 * hf;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int64_t t = tq + (int64_t)(32 * db + col) * Tq32 + r0;
        const bf16x8_t oh = ld_perm(op.OTh + t), ol = ld_perm(op.OTl + t);
        const bf16x8_t qh = ld_perm(op.QTh + t), ql = ld_perm(op.QTl + t);
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
    for (int e = tid; e < 32 * (D / 2); e += THREADS) {
      const int kk = e / (D / 2), pr = e % (D / 2);
      const int kg = k0 + kk;
      if (kg >= nkb) continue;
      float g1 = 0.f, g2 = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) { g1 += part[w][kk][pr]; g2 += part[w][kk][pr + 64]; }
      float* o;
      if (pass == 0) {
        o = kg < M ? dVmem + (((int64_t)b * Mmax + kg) * Hkv + g) * D : dVloc + (((int64_t)b * Tl + kg - M) * Hkv + g) * D;
      } else {
        g1 *= scale;
        g2 *= scale;
        if (kg < M) {
          o = dKmem + (((int64_t)b * Mmax + kg) * Hkv + g) * D;
        } else {
          float c, s;
          rope_cs(rope_offset + (kg - M), rr.rev[pr], &c, &s);
          const float y1 = g1 * c + g2 * s, y2 = g2 * c - g1 * s;
          g1 = y1;
          g2 = y2;
          o = dKloc + (((int64_t)b * Tl + kg - M) * Hkv + g) * D;
        }
      }
      o[pr] = g1;
      o[pr + 64] = g2;
    }
  }
}

struct BwdLayout {
  int Tq32, NK;
  size_t q[8], k[5], lse, dlt, total;
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
                    float* dQ, float* dKloc, float* dVloc, float* dKmem, float* dVmem, void* workspace,
                    hipStream_t stream) {
  const BwdLayout L = layout(B, Tq, Hq, Tl, Hkv, Mmax);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  uint16_t* qa[8];
  uint16_t* ka[5];
  for (int i = 0; i < 8; ++i) qa[i] = reinterpret_cast<uint16_t*>(ws + L.q[i]);
  for (int i = 0; i < 5; ++i) ka[i] = reinterpret_cast<uint16_t*>(ws + L.k[i]);
  float* lse = reinterpret_cast<float*>(ws + L.lse);
  float* dlt = reinterpret_cast<float*>(ws + L.dlt);
  RopeRev rr;
  const double two_pi = 6.283185307179586;
  for (int i = 0; i < D / 2; ++i) rr.rev[i] = pow(rope_base, -2.0 * i / D) / two_pi;
  const float scale_log2e = scale * 1.4426950408889634f;

  hipLaunchKernelGGL(bwd_prep_q_kernel, dim3((unsigned)L.Tq32, (unsigned)Hq, (unsigned)B), dim3(64), 0, stream, Q,
                     dO, Tq, L.Tq32, Hq, Tl, rope_offset, rr, qa[0], qa[1], qa[2], qa[3], qa[4], qa[5], qa[6], qa[7]);
  MSA_CHECK_LAUNCH();
  hipLaunchKernelGGL(bwd_prep_k_kernel, dim3((unsigned)L.NK, (unsigned)Hkv, (unsigned)B), dim3(64), 0, stream, Kloc,
                     Vloc, Tl, Hkv, Kmem, Vmem, mem_entry_stride, Mmax, mem_len, L.NK, rope_offset, rr, ka[0], ka[1],
                     ka[2], ka[3], ka[4], dKmem, dVmem);
  MSA_CHECK_LAUNCH();
  const Ops op{qa[0], qa[1], qa[2], qa[3], qa[4], qa[5], qa[6], qa[7], ka[0], ka[1], ka[2], ka[3], ka[4]};
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)(L.Tq32 / 32), (unsigned)Hq, (unsigned)B), dim3(THREADS), 0,
                     stream, op, mem_len, Tq, L.Tq32, Hq, Tl, Hkv, Mmax, L.NK, rope_offset, rr, scale_log2e, scale, lse,
                     dlt, dQ);
  MSA_CHECK_LAUNCH();
  hipLaunchKernelGGL(bwd_dkv_kernel, dim3((unsigned)(L.NK / 32), (unsigned)Hkv, (unsigned)B), dim3(THREADS), 0,
                     stream, op, mem_len, Tq, L.Tq32, Hq, Tl, Hkv, Mmax, L.NK, rope_offset, rr, scale_log2e, scale,
                     lse, dlt, dKloc, dVloc, dKmem, dVmem);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

}  // namespace msa
