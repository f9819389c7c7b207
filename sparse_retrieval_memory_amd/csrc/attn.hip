// Sparse attention over [pooled memory ++ causal local KV] (medium write-up
// sec. 2 and b-lab.team summary sec. 1: the selected documents' compressed
// K/V are concatenated with the query's local K/V for autoregressive
// decoding; b-lab.team sec. 1, Global RoPE: the query's start index is offset
// by k, the number of retrieved blocks).
//
// Flash-style, fp32 throughout: one workgroup owns 16 query rows of one q-head
// and streams keys in LDS tiles of 64 (memory entries first, then local keys,
// stopping at the causal limit of its last row), keeping a running max, sum
// and output per row (online softmax).  Query rows and local keys are rotated
// here, with angles computed in fp64; memory keys arrive already rotated.
// Scores are pre-scaled by log2(e) so the exponentials are exp2.
#include "msa_internal.h"

#include <math.h>

namespace msa {
namespace {

constexpr int D = 128;
constexpr int RQ = 16;     // query rows per workgroup
constexpr int KT = 64;     // keys per tile
constexpr int THREADS = 256;
constexpr int KSTR = D + 4;  // padded LDS row (floats) for keys

__device__ __forceinline__ void load_bf16x8(const uint16_t* p, float* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
  out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
  out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
  out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
}

// cos/sin of pos * base^(-2i/D), evaluated in fp64
__device__ __forceinline__ void rope_cs(double pos, int i, double log2_base, float* c, float* s) {
  const double theta = exp2(-(2.0 * i / D) * log2_base);
  double sn, cs;
  sincos(pos * theta, &sn, &cs);
  *c = (float)cs;
  *s = (float)sn;
}

__global__ void __launch_bounds__(THREADS, 2)
attn_kernel(const uint16_t* __restrict__ Q, int Tq, int Hq, const uint16_t* __restrict__ Kloc,
            const uint16_t* __restrict__ Vloc, int Tl, int Hkv, const uint16_t* __restrict__ Kmem,
            const uint16_t* __restrict__ Vmem, int64_t mstride, int Mmax,
            const int32_t* __restrict__ mem_len, int rope_offset, double log2_base, float scale_log2e,
            float* __restrict__ O) {
  __shared__ __attribute__((aligned(16))) float qs[RQ][D];
  __shared__ __attribute__((aligned(16))) float ks[KT][KSTR];
  __shared__ __attribute__((aligned(16))) float vs[KT][D];
  __shared__ __attribute__((aligned(16))) float ps[RQ][KT];

  const int tid = threadIdx.x;
  const int row0 = blockIdx.x * RQ;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int g = h / (Hq / Hkv);
  int M = mem_len[b];
  if (M < 0) M = 0;
  if (M > Mmax) M = Mmax;

  // --- query rows: rotate at rope_offset + (Tl - Tq) + i, pre-scale
  for (int x = tid; x < RQ * (D / 2); x += THREADS) {
    const int r = x / (D / 2), i = x % (D / 2);
    const int qi = row0 + r;
    float a = 0.f, c2 = 0.f;
    if (qi < Tq) {
      const uint16_t* q = Q + (((int64_t)b * Tq + qi) * Hq + h) * D;
      const float x1 = __uint_as_float((uint32_t)q[i] << 16);
      const float x2 = __uint_as_float((uint32_t)q[i + D / 2] << 16);
      float c, s;
      rope_cs((double)(rope_offset + (Tl - Tq) + qi), i, log2_base, &c, &s);
      a = (x1 * c - x2 * s) * scale_log2e;
      c2 = (x2 * c + x1 * s) * scale_log2e;
    }
    qs[r][i] = a;
    qs[r][i + D / 2] = c2;
  }

  // per-thread roles
  const int sr = tid / 16;          // score row / output row
  const int sc = tid % 16;          // score key column (keys sc + 16 j)
  const int od = (tid % 16) * 8;    // output dims [od, od + 8)
  float m_run = -INFINITY, l_run = 0.f;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;

  // keys this workgroup needs: all memory + local keys up to the causal limit of its last row
  int last_row = row0 + RQ - 1;
  if (last_row > Tq - 1) last_row = Tq - 1;
  const int n_local = (Tl - Tq) + last_row + 1;   // local keys 0..n_local-1
  const int n_keys = M + n_local;
  const int64_t mem_base = (int64_t)b * Mmax;

  for (int k0 = 0; k0 < n_keys; k0 += KT) {
    __syncthreads();   // previous tile fully consumed (and qs visible on the first pass)
    // load K and V tile: thread -> key tid / 4, quarter tid % 4
    {
      const int kk = tid >> 2, qd = tid & 3;
      const int j = k0 + kk;
      float kx[32], vx[32];
      if (j < n_keys) {
        const uint16_t *kp, *vp;
        if (j < M) {
          kp = Kmem + (mem_base + j) * mstride + (int64_t)g * D;
          vp = Vmem + (mem_base + j) * mstride + (int64_t)g * D;
        } else {
          const int jl = j - M;
          kp = Kloc + (((int64_t)b * Tl + jl) * Hkv + g) * D;
          vp = Vloc + (((int64_t)b * Tl + jl) * Hkv + g) * D;
        }
        load_bf16x8(kp + 16 * qd, kx);
        load_bf16x8(kp + 16 * qd + 8, kx + 8);
        load_bf16x8(kp + 64 + 16 * qd, kx + 16);
        load_bf16x8(kp + 64 + 16 * qd + 8, kx + 24);
        load_bf16x8(vp + 32 * qd, vx);
        load_bf16x8(vp + 32 * qd + 8, vx + 8);
        load_bf16x8(vp + 32 * qd + 16, vx + 16);
        load_bf16x8(vp + 32 * qd + 24, vx + 24);
        if (j >= M) {
          const double pos = (double)(rope_offset + (j - M));
#pragma unroll 4
          for (int e = 0; e < 16; ++e) {
            float c, s;
            rope_cs(pos, 16 * qd + e, log2_base, &c, &s);
            const float x1 = kx[e], x2 = kx[16 + e];
            kx[e] = x1 * c - x2 * s;
            kx[16 + e] = x2 * c + x1 * s;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) { kx[e] = 0.f; vx[e] = 0.f; }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        ks[kk][16 * qd + e] = kx[e];
        ks[kk][64 + 16 * qd + e] = kx[16 + e];
      }
#pragma unroll
      for (int e = 0; e < 32; e += 4)
        *reinterpret_cast<float4*>(&vs[kk][32 * qd + e]) = make_float4(vx[e], vx[e + 1], vx[e + 2], vx[e + 3]);
    }
    __syncthreads();

    // scores for row sr, keys sc + 16 jj
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
    for (int d = 0; d < D; d += 4) {
      const float4 q = *reinterpret_cast<const float4*>(&qs[sr][d]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 kv = *reinterpret_cast<const float4*>(&ks[sc + 16 * jj][d]);
        s4[jj] = fmaf(q.x, kv.x, s4[jj]);
        s4[jj] = fmaf(q.y, kv.y, s4[jj]);
        s4[jj] = fmaf(q.z, kv.z, s4[jj]);
        s4[jj] = fmaf(q.w, kv.w, s4[jj]);
      }
    }
    const int qi = row0 + sr;
    const int lim = (Tl - Tq) + qi;   // last visible local key of this row
    float tmax = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = k0 + sc + 16 * jj;
      bool vis = j < n_keys && qi < Tq;
      if (j >= M) vis = vis && (j - M) <= lim;
      s4[jj] = vis ? s4[jj] : -INFINITY;
      tmax = fmaxf(tmax, s4[jj]);
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float lsum = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float pj = (m_new == -INFINITY) ? 0.f : exp2f(s4[jj] - m_new);
      ps[sr][sc + 16 * jj] = pj;
      lsum += pj;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) lsum += __shfl_xor(lsum, off);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    __syncthreads();

#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
    for (int j = 0; j < KT; ++j) {
      const float pj = ps[sr][j];
      const float4 v0 = *reinterpret_cast<const float4*>(&vs[j][od]);
      const float4 v1 = *reinterpret_cast<const float4*>(&vs[j][od + 4]);
      o[0] = fmaf(pj, v0.x, o[0]); o[1] = fmaf(pj, v0.y, o[1]);
      o[2] = fmaf(pj, v0.z, o[2]); o[3] = fmaf(pj, v0.w, o[3]);
      o[4] = fmaf(pj, v1.x, o[4]); o[5] = fmaf(pj, v1.y, o[5]);
      o[6] = fmaf(pj, v1.z, o[6]); o[7] = fmaf(pj, v1.w, o[7]);
    }
  }

  const int qi = row0 + sr;
  if (qi < Tq) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* out = O + (((int64_t)b * Tq + qi) * Hq + h) * D + od;
    *reinterpret_cast<float4*>(out) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    *reinterpret_cast<float4*>(out + 4) = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
  }
}

}  // namespace

int launch_attn(const uint16_t* Q, int B, int Tq, int Hq, const uint16_t* Kloc, const uint16_t* Vloc,
                int Tl, int Hkv, const uint16_t* Kmem, const uint16_t* Vmem, int64_t mem_entry_stride,
                int Mmax, const int32_t* mem_len, int rope_offset, double rope_base, float scale,
                float* O, hipStream_t stream) {
  dim3 grid((unsigned)((Tq + RQ - 1) / RQ), (unsigned)Hq, (unsigned)B);
  const float scale_log2e = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(attn_kernel, grid, dim3(THREADS), 0, stream, Q, Tq, Hq, Kloc, Vloc, Tl, Hkv, Kmem,
                     Vmem, mem_entry_stride, Mmax, mem_len, rope_offset, log2(rope_base), scale_log2e, O);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

}  // namespace msa
