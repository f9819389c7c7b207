// Backward of the routing scores: gradients w.r.t. the router queries and the
// selected chunks' pooled router keys, given the gradient of the document scores.
//
// b-lab.team summary sec. 2 (training): an auxiliary routing loss supervises the
// sparse attention towards the right evidence; chatpaper.ai Abstract: MSA is
// trained end to end.  The forward (route.hip) is a head mean of cosines, a max
// over query tokens, then a max over a document's chunks.  Readings: each max
// passes its gradient to its first (lowest-index) maximiser; an excluded or empty
// document, a zero upstream gradient or a zero vector passes nothing.  With
// q^ = q/|q|, k^ = k/|k| and c = q^.k^ per head:
//   dc/dq = (k^ - c q^) / |q|,     dc/dk = (q^ - c k^) / |k|.
//
// Kernels, in launch order:
//   route_bwd_select_kernel<H>  32 documents of one query per workgroup (8
//       lanes each).  The selected chunk is the first maximum of the forward's
//       chunk scores; the 32 chunk rows are staged in LDS (64 KB at H = 8, so two
//       workgroups share a CU) and the token scores S[t] = mean_h cos are
//       recomputed on v_mfma_f32_32x32x16_bf16 (router rows as A, the chunk rows
//       as the 32 B columns) to find the first maximising token.  Then per
//       document and head: the cosine, the key-gradient row, and two weights of
//       the query gradient (w/|k| and w c, w = dL/d doc / H).
//   hist / scan / scatter  a stable counting sort of the documents by selected
//       token (tiles of 1,024 documents), so each token's documents sit
//       contiguously and in document order.
//   piece<H>  each token's list is cut into pieces of 64 documents (the scan
//       writes each piece's first position and count; the scatter writes the
//       sorted documents' chunk ids next to them, so a piece's row loads wait on
//       two lookups only); one workgroup sums w/|k| * k and w c over a piece
//       (16-byte row loads, 16 in flight per lane, rows split over lane groups
//       and added in a fixed order).
//   final   one workgroup per token adds its pieces in order:
//       dq = (sum w k/|k| - q^ sum w c) / |q|.  No atomics: the result does not
//       depend on scheduling.
#include "msa_internal.h"

#include <math.h>

namespace msa {
namespace {

constexpr int D = 128;
constexpr int SEL_DOCS = 32;        // documents per select workgroup (the 32 MFMA B columns)
constexpr int SEL_THREADS = 256;    // 4 waves; wave w takes token tiles w, w + 4, ...
constexpr int LPD = SEL_THREADS / SEL_DOCS;   // lanes per document
constexpr int SORT_TILE = 1024;     // documents per histogram / scatter workgroup
constexpr int PIECE = 64;           // documents per partial sum of the query gradient
constexpr int PIECE_UNROLL = 16;
constexpr int MAX_T = ROUTE_BWD_MAX_T;

template <int H>
struct SelCfg {
  static constexpr int HD = H * D;
  static constexpr int KROW = HD + 8;     // staged row stride (bf16): +16 B staggers the banks by 4
  static constexpr int VPR = HD / 8;      // 16-byte vectors per chunk row
};

__device__ __forceinline__ float sq_norm_piece(uint4 v, float acc) {
  acc = dot2_bf16(v.x, v.x, acc);
  acc = dot2_bf16(v.y, v.y, acc);
  acc = dot2_bf16(v.z, v.z, acc);
  acc = dot2_bf16(v.w, v.w, acc);
  return acc;
}
__device__ __forceinline__ float inv_norm(float ss) { return ss > 0.f ? 1.0f / sqrtf(ss) : 0.f; }

// (score, token) -> key whose maximum is the largest score, then the lowest token.
__device__ __forceinline__ uint64_t argmax_key(float s, int t) {
  return ((uint64_t)enc_f32(s) << 32) | (uint32_t)(0x7FFFFFFF - t);
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// The fp32 key-gradient rows are written once and not read again here: streaming
// (non-temporal) stores keep them from sitting dirty in L2 / Infinity Cache, where
// their write-back would otherwise slow the later kernels' reads.
__device__ __forceinline__ void nt_store4(float4* p, float a, float b, float c, float d) {
  __builtin_nontemporal_store((f32x4_t){a, b, c, d}, reinterpret_cast<f32x4_t*>(p));
}

// Sum over each row of 16 lanes, every lane receiving the total: lane swaps within
// quads (quad_perm [1,0,3,2], [2,3,0,1]), then across the quads of a half-row
// (row_half_mirror) and across the halves (row_mirror), all DPP moves.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}

template <int H>
__global__ void __launch_bounds__(SEL_THREADS, 2)
route_bwd_select_kernel(const uint16_t* __restrict__ Qr, int T, const uint16_t* __restrict__ Krbar,
                        const float* __restrict__ knorm, const int64_t* __restrict__ off, int64_t n_docs,
                        int64_t n_chunks, const uint8_t* __restrict__ exclude, const float* __restrict__ chunk_scores,
                        const float* __restrict__ dDoc, float* __restrict__ dK, int32_t* __restrict__ sel,
                        float* __restrict__ ikw, float* __restrict__ wcos) {
  using CF = SelCfg<H>;
  __shared__ __attribute__((aligned(16))) uint16_t k_s[SEL_DOCS * CF::KROW];
  __shared__ float ik_s[SEL_DOCS][H];
  __shared__ __attribute__((aligned(16))) float iq_s[SEL_THREADS / 64][32];
  __shared__ uint64_t best_s[SEL_THREADS / 64][SEL_DOCS];
  __shared__ int64_t g_s[SEL_DOCS];
  __shared__ int t_s[SEL_DOCS];
  __shared__ int any_s;

  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, m = lane & 31;
  const int idoc = tid / LPD, sub = tid % LPD;
  const int64_t d = (int64_t)blockIdx.x * SEL_DOCS + idoc;
  const int64_t bd = (int64_t)b * n_docs + d;
  const bool in = d < n_docs;

  // ---- selected chunk: first maximum of the document's chunk scores, LPD lanes per document
  if (tid == 0) any_s = 0;
  float dd = 0.f;
  int64_t c0 = 0;
  uint64_t key = 0;                   // (score, -chunk within the document); 0 = none
  if (in) {
    dd = dDoc[bd];
    if (!(exclude && exclude[bd]) && dd != 0.f) {
      c0 = off[d];
      const int64_t c1 = off[d + 1];
      for (int64_t c = c0 + sub; c < c1; c += LPD)
        key = max_u64(key, ((uint64_t)enc_f32(chunk_scores[(int64_t)b * n_chunks + c]) << 32) |
                               (uint32_t)(0xFFFFFFFFu - (uint32_t)(c - c0)));
    }
  }
#pragma unroll
  for (int s = 1; s < LPD; s <<= 1) key = max_u64(key, shfl_xor_u64(key, s));
  __syncthreads();
  if (sub == 0) {
    const int64_t g = key ? c0 + (int64_t)(0xFFFFFFFFu - (uint32_t)key) : -1;
    g_s[idoc] = g;
    if (g >= 0) any_s = 1;
  }
  __syncthreads();

  uint64_t bk = 0;                    // best token key of column m
  if (any_s) {
    // ---- stage the selected rows (zeros for documents without one), all loads in flight
    constexpr int NV = SEL_DOCS * CF::VPR / SEL_THREADS;
    uint4 v[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int x = tid + u * SEL_THREADS;
      const int64_t g = g_s[x / CF::VPR];
      v[u] = make_uint4(0, 0, 0, 0);
      if (g >= 0) v[u] = *reinterpret_cast<const uint4*>(Krbar + g * CF::HD + 8 * (x % CF::VPR));
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int x = tid + u * SEL_THREADS;
      *reinterpret_cast<uint4*>(&k_s[(x / CF::VPR) * CF::KROW + 8 * (x % CF::VPR)]) = v[u];
    }
    __syncthreads();
    if (tid < SEL_DOCS * H) {
      const int i = tid / H, h = tid % H;
      const int64_t g = g_s[i];
      float ik = 0.f;
      if (g >= 0) {
        if (knorm) {
          ik = knorm[g * H + h];
        } else {
          float ss = 0.f;
          for (int x = 0; x < D / 8; ++x)
            ss = sq_norm_piece(*reinterpret_cast<const uint4*>(&k_s[i * CF::KROW + h * D + 8 * x]), ss);
          ik = inv_norm(ss);
        }
      }
      ik_s[i][h] = ik;
    }
    __syncthreads();

    // ---- token scores of the selected chunks: 32 tokens x 32 chunks per wave step
    const int n_tt = (T + 31) / 32;
    const float inv_h = 1.0f / (float)H;
    for (int tt = wave; tt < n_tt; tt += SEL_THREADS / 64) {
      const int t = tt * 32 + m;
      const bool tv = t < T;
      const uint16_t* qrow = Qr + ((int64_t)b * T + (tv ? t : 0)) * CF::HD + 8 * half;
      bf16x8_t a[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (tv) x = *reinterpret_cast<const uint4*>(qrow + 16 * ks);
        a[ks] = __builtin_bit_cast(bf16x8_t, x);
      }
      f32x16_t s0 = {};
#pragma unroll 2
      for (int h = 0; h < H; ++h) {
        bf16x8_t an[8];
        if (h + 1 < H) {
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (tv) x = *reinterpret_cast<const uint4*>(qrow + (h + 1) * D + 16 * ks);
            an[ks] = __builtin_bit_cast(bf16x8_t, x);
          }
        }
        float ss = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) ss = sq_norm_piece(__builtin_bit_cast(uint4, a[ks]), ss);
        ss += __shfl_xor(ss, 32);
        f32x16_t c = {};
        const uint16_t* bp = &k_s[m * CF::KROW + h * D + 8 * half];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], *reinterpret_cast<const bf16x8_t*>(bp + 16 * ks), c,
                                                      0, 0, 0);
        // the row (token) inverse norms of this head, through a wave-private LDS slot
        if (half == 0) iq_s[wave][m] = inv_norm(ss);
        __builtin_amdgcn_wave_barrier();
        const float ik = ik_s[m][h];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t r = *reinterpret_cast<const f32x4_t*>(&iq_s[wave][8 * q + 4 * half]);
#pragma unroll
          for (int e = 0; e < 4; ++e) s0[4 * q + e] += c[4 * q + e] * r[e] * ik;
        }
        __builtin_amdgcn_wave_barrier();
        if (h + 1 < H) {
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) a[ks] = an[ks];
        }
      }
      // C register i holds row 8 (i / 4) + 4 half + i % 4 of column m
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tok = tt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        if (tok < T) bk = max_u64(bk, argmax_key(s0[i] * inv_h, tok));
      }
    }
    bk = max_u64(bk, shfl_xor_u64(bk, 32));
  }
  if (half == 0) best_s[wave][m] = bk;
  __syncthreads();
  if (tid < SEL_DOCS) {
    uint64_t bb = 0;
#pragma unroll
    for (int w = 0; w < SEL_THREADS / 64; ++w) bb = max_u64(bb, best_s[w][tid]);
    const bool ok = g_s[tid] >= 0 && bb != 0;      // every valid token has a nonzero key
    t_s[tid] = ok ? 0x7FFFFFFF - (int)(uint32_t)bb : -1;
    if (!ok) g_s[tid] = -1;
  }
  __syncthreads();

  // ---- per document (LPD lanes) and head: cosine, key gradient, query-gradient weights
  if (!in) return;
  const int64_t g = g_s[idoc];
  const int tsel = t_s[idoc];
  if (sub == 0) {
    sel[2 * bd] = (int32_t)g;
    sel[2 * bd + 1] = tsel;
  }
  float4* o = reinterpret_cast<float4*>(dK + bd * CF::HD);
  if (g < 0) {
#pragma unroll
    for (int x = sub; x < CF::HD / 4; x += LPD) nt_store4(o + x, 0.f, 0.f, 0.f, 0.f);
    if (sub < H) { ikw[bd * H + sub] = 0.f; wcos[bd * H + sub] = 0.f; }
    return;
  }
  const float w = dd * (1.0f / (float)H);
  const uint16_t* qrow = Qr + ((int64_t)b * T + tsel) * CF::HD;
  const uint16_t* krow = &k_s[idoc * CF::KROW];
  uint2 qv[H][4];
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) qv[h][j] = *reinterpret_cast<const uint2*>(qrow + h * D + 4 * (sub + LPD * j));
  float my_ikw = 0.f, my_wc = 0.f;
#pragma unroll
  for (int h = 0; h < H; ++h) {
    uint2 kv[4];
    float qq = 0.f, kk = 0.f, qk = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kv[j] = *reinterpret_cast<const uint2*>(krow + h * D + 4 * (sub + LPD * j));
      qq = dot2_bf16(qv[h][j].x, qv[h][j].x, qq); qq = dot2_bf16(qv[h][j].y, qv[h][j].y, qq);
      kk = dot2_bf16(kv[j].x, kv[j].x, kk); kk = dot2_bf16(kv[j].y, kv[j].y, kk);
      qk = dot2_bf16(qv[h][j].x, kv[j].x, qk); qk = dot2_bf16(qv[h][j].y, kv[j].y, qk);
    }
#pragma unroll
    for (int s = 1; s < LPD; s <<= 1) {
      qq += __shfl_xor(qq, s);
      kk += __shfl_xor(kk, s);
      qk += __shfl_xor(qk, s);
    }
    float ca = 0.f, cb = 0.f, ik = 0.f, cs = 0.f;
    if (qq > 0.f && kk > 0.f) {
      const float iq = 1.0f / sqrtf(qq);
      ik = 1.0f / sqrtf(kk);
      cs = qk * iq * ik;
      ca = w * ik * iq;        // dK = w (q^ - c k^) / |k| = ca q - cb k
      cb = w * ik * ik * cs;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      nt_store4(o + h * (D / 4) + sub + LPD * j, ca * bf16_lo(qv[h][j].x) - cb * bf16_lo(kv[j].x),
                ca * bf16_hi(qv[h][j].x) - cb * bf16_hi(kv[j].x), ca * bf16_lo(qv[h][j].y) - cb * bf16_lo(kv[j].y),
                ca * bf16_hi(qv[h][j].y) - cb * bf16_hi(kv[j].y));
    if (h == sub) { my_ikw = w * ik; my_wc = w * cs; }
  }
  if (sub < H) { ikw[bd * H + sub] = my_ikw; wcos[bd * H + sub] = my_wc; }
}

// ---------------------------------------------------------------- H = 8 path
// The selected chunk of every document (first maximum of its chunk scores),
// LPD lanes per document; -1 for a document that passes no gradient.
__global__ void __launch_bounds__(256)
route_bwd_pick_kernel(const int64_t* __restrict__ off, int64_t n_docs, int64_t n_chunks,
                      const uint8_t* __restrict__ exclude, const float* __restrict__ chunk_scores,
                      const float* __restrict__ dDoc, int64_t* __restrict__ gsel) {
  const int b = blockIdx.y;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t d = gid / LPD;
  const int sub = (int)(gid % LPD);
  uint64_t key = 0;
  int64_t c0 = 0;
  if (d < n_docs) {
    const int64_t bd = (int64_t)b * n_docs + d;
    if (!(exclude && exclude[bd]) && dDoc[bd] != 0.f) {
      c0 = off[d];
      const int64_t c1 = off[d + 1];
      for (int64_t c = c0 + sub; c < c1; c += LPD)
        key = max_u64(key, ((uint64_t)enc_f32(chunk_scores[(int64_t)b * n_chunks + c]) << 32) |
                               (uint32_t)(0xFFFFFFFFu - (uint32_t)(c - c0)));
    }
  }
#pragma unroll
  for (int s = 1; s < LPD; s <<= 1) key = max_u64(key, shfl_xor_u64(key, s));
  if (sub == 0 && d < n_docs)
    gsel[(int64_t)b * n_docs + d] = key ? c0 + (int64_t)(0xFFFFFFFFu - (uint32_t)key) : -1;
}

constexpr int PG = 32;                       // documents per group of the persistent kernel
constexpr int SELECT8_WORKGROUPS = 256;      // one per CU
constexpr int P_HD = 8 * D;
constexpr int P_KROW = P_HD + 8;             // staged row stride (bf16): banks staggered by 4

__device__ __forceinline__ int64_t shfl_i64(int64_t v, int src) {
  const int lo = __shfl((int)(uint32_t)v, src), hi = __shfl((int)(uint32_t)((uint64_t)v >> 32), src);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

constexpr int S8_WAVES = 8;                  // 4 token tiles x 2 head groups
constexpr int S8_THREADS = 64 * S8_WAVES;

// Copies into LDS for the persistent select kernel, written as inline assembly: the compiler does
// not track them, so it neither orders later LDS reads behind them nor counts them in the waits of
// the group's own loads; the group loop waits for them with an explicit count instead.  Each copy
// only reads its operands (no register is written), and M0 is set right before it.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
// raw buffer resource on `base` covering `bytes` (reads past them return 0); wave-uniform values
__device__ __forceinline__ i32x4_t copy_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r[0] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);   // stride 0
  r[2] = (int32_t)__builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000;
  return r;
}
__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)lds);
}
// 16 bytes a lane: lane i reads the resource at voff and writes lds + 16 i
__device__ __forceinline__ void copy16_buf(const i32x4_t& rs, uint32_t voff, const void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_addr(lds)), "v"(voff), "s"(rs) : "memory", "m0");
}
// 4 bytes a lane: lane i reads the resource at voff and writes lds + 4 i
__device__ __forceinline__ void copy4_buf(const i32x4_t& rs, uint32_t voff, const void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds_addr(lds)), "v"(voff), "s"(rs) : "memory", "m0");
}
// 4 bytes a lane from its own address: lane i reads *gptr and writes lds + 4 i
__device__ __forceinline__ void copy4_addr(const void* gptr, const void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds_addr(lds)), "v"(gptr) : "memory", "m0");
}

// Copies for one group: its selected rows into `rows` (wave w: documents 4w .. 4w+3, one 1 KB
// half-row per copy) and, with stored norms, their 1/|k| into `ik` (waves 0-3: lane l of wave w
// takes entry 64 w + l, i.e. document (64 w + l) / 8, head l % 8).  gv: lanes 0..31 hold the
// group's chunk ids.  A document with id -1 gets zero rows and chunk 0's norms (none at all when the
// store is empty); its scores are discarded.
__device__ __forceinline__ void copy_group(const uint16_t* __restrict__ Krbar, const float* __restrict__ knorm,
                                           int64_t n_chunks, int64_t gv, uint16_t* rows, float* ik, int wave,
                                           int lane, uint32_t voff16) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int doc = wave * 4 + (q >> 1), hh = q & 1;
    // the document's id straight into scalar registers (the lane is wave-uniform)
    const int64_t g = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)((uint64_t)gv >> 32), doc) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)gv, doc));
    copy16_buf(copy_rsrc(Krbar + (g >= 0 ? g : 0) * P_HD + hh * 512, g >= 0 ? 1024u : 0u), voff16,
               rows + doc * P_KROW + hh * 512);
  }
  if (knorm && n_chunks > 0 && wave < 4) {
    const int e = wave * 64 + lane;
    const int64_t g = shfl_i64(gv, e >> 3);
    copy4_addr(knorm + (g >= 0 ? g : 0) * 8 + (e & 7), ik + wave * 64);
  }
}

// Chunk ids of group `gr` (32 int64, 256 B) into `ids`: one 4-byte copy by the last wave.  Entries
// past the last document read 0 (the resource's range); group_ids masks them.
__device__ __forceinline__ void copy_ids(const int64_t* __restrict__ gs, int64_t n_docs, int64_t gr, int64_t* ids,
                                         int wave, uint32_t voff4) {
  if (wave == S8_WAVES - 1) {
    const int64_t first = gr * PG;
    const int64_t left = first < n_docs ? n_docs - first : 0;
    copy4_buf(copy_rsrc(gs + (left > 0 ? first : 0), (uint32_t)((left < PG ? left : PG) * 8)), voff4, ids);
  }
}
// lanes 0..31: the chunk id of document gr * 32 + lane from the copied ids (-1 past the end)
__device__ __forceinline__ int64_t group_ids(const int64_t* ids, int64_t gr, int64_t n_docs, int lane) {
  const int64_t d = gr * PG + (lane & 31);
  const int64_t v = ids[lane & 31];
  return (lane < 32 && d < n_docs) ? v : -1;
}

// Router rows of token tile tt as A operands for heads 4 hg .. 4 hg + 3, and their
// inverse norms per head.
__device__ __forceinline__ void load_rows4(const uint16_t* __restrict__ Qr, int b, int T, int tt, int hg, int m,
                                           int half, bf16x8_t (&a)[4][8], float (*iq)[32]) {
  const int t = tt * 32 + m;
  const bool tv = t < T;
  const uint16_t* qrow = Qr + ((int64_t)b * T + (tv ? t : 0)) * P_HD + hg * 4 * D + 8 * half;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (tv) x = *reinterpret_cast<const uint4*>(qrow + h * D + 16 * ks);
      a[h][ks] = __builtin_bit_cast(bf16x8_t, x);
      ss = sq_norm_piece(x, ss);
    }
    ss += __shfl_xor(ss, 32);
    if (half == 0) iq[h][m] = inv_norm(ss);
  }
  __builtin_amdgcn_wave_barrier();
}

struct S8Lds {
  float ik[2][PG][8];                  // 1/|k| of (document, head), one per row buffer
  int64_t ids[2][PG];                  // chunk ids, copied two groups ahead
  float iq[S8_WAVES][4][32];
  f32x4_t xchg[4][64 * 4];             // head group 1's partial scores, per token tile
  uint64_t best[4][PG];
  int tsel[PG];
};

// One group of 32 documents whose rows sit in `cur` and norms in `ik_cur`; the next group's
// copies go into `nxt` / `ik_nxt` meanwhile, and the chunk ids of the group after it into
// `ids_wr`.  g_cur (lanes 0..31): this group's chunk ids on entry, the next group's on exit.
// RESIDENT (T <= 128): the router rows stay in `a` for the whole kernel; else each token tile's
// rows are loaded per round.
template <bool RESIDENT>
__device__ __forceinline__ void select8_group(const uint16_t* __restrict__ Qr, int b, int T,
                                              const uint16_t* __restrict__ Krbar, const float* __restrict__ knorm,
                                              int64_t n_chunks, int64_t n_docs, const float* __restrict__ dDoc,
                                              const int64_t* __restrict__ gs, int64_t grp, int64_t stride,
                                              int64_t& g_cur, bool first, const uint16_t* cur, uint16_t* nxt,
                                              float* ik_cur, float* ik_nxt, const int64_t* ids_rd, int64_t* ids_wr,
                                              bf16x8_t (&a)[4][8], S8Lds& sm,
                                              float* __restrict__ dK, int32_t* __restrict__ sel,
                                              float* __restrict__ ikw, float* __restrict__ wcos, int tid, int wave,
                                              int lane, uint32_t voff16, uint32_t voff4) {
  constexpr int H = 8;
  const int half = lane >> 5, m = lane & 31;
  const int rt = wave & 3, hg = wave >> 2;         // token tile slot, head group
  // This wave's copies for this group: the prologue's (first group: wait for everything), else
  // those issued at the previous group's start.  The previous group was not the last one, so all
  // its documents exist and this wave issued its 16 key-gradient stores after those copies: they
  // may stay in flight (vector memory completes in order).
  if (first)
    __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
  else
    __builtin_amdgcn_s_waitcnt(0x4F70);            // vmcnt(16)
  asm volatile("" ::: "memory");
  lds_barrier();                                   // everyone's copies landed; the previous group is done with `nxt`
  const int64_t nx = grp + stride;
  const int64_t g_nxt = group_ids(ids_rd, nx, n_docs, lane);
  copy_group(Krbar, knorm, n_chunks, g_nxt, nxt, ik_nxt, wave, lane, voff16);
  copy_ids(gs, n_docs, nx + stride, ids_wr, wave, voff4);
  if (!knorm && tid < PG * H) {
    // 1/|k| of (document tid % 32, head tid / 32) from the staged rows (consecutive lanes on
    // consecutive rows: no bank conflicts)
    const int doc = tid & 31, h = tid >> 5;
    float ss = 0.f;
#pragma unroll
    for (int x = 0; x < D / 8; ++x)
      ss = sq_norm_piece(*reinterpret_cast<const uint4*>(cur + doc * P_KROW + h * D + 8 * x), ss);
    ik_cur[doc * 8 + h] = inv_norm(ss);
  }
  lds_barrier();
  // token scores of the 32 rows: wave (rt, hg) takes token tiles rt, rt + 4, ... over heads 4 hg ..
  uint64_t bk = 0;
  const int n_tt = (T + 31) / 32;
  const float inv_h = 1.0f / (float)H;
  const int n_rounds = (n_tt + 3) / 4;
  for (int rd = 0; rd < n_rounds; ++rd) {
    const int tt = rd * 4 + rt;
    const bool act = tt < n_tt;
    f32x16_t s0 = {};
    if (act) {
      if constexpr (!RESIDENT) load_rows4(Qr, b, T, tt, hg, m, half, a, sm.iq[wave]);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        f32x16_t c = {};
        const uint16_t* bp = cur + m * P_KROW + (hg * 4 + h) * D + 8 * half;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[h][ks], *reinterpret_cast<const bf16x8_t*>(bp + 16 * ks),
                                                      c, 0, 0, 0);
        const float ik = ik_cur[m * 8 + hg * 4 + h];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t r = *reinterpret_cast<const f32x4_t*>(&sm.iq[wave][h][8 * q + 4 * half]);
#pragma unroll
          for (int e = 0; e < 4; ++e) s0[4 * q + e] += c[4 * q + e] * r[e] * ik;
        }
      }
    }
    // head group 1 hands its partial sums to head group 0 (same token tile)
    if (hg == 1 && act) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sm.xchg[rt][lane * 4 + q] = (f32x4_t){s0[4 * q], s0[4 * q + 1], s0[4 * q + 2], s0[4 * q + 3]};
    }
    lds_barrier();
    if (hg == 0 && act) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t x = sm.xchg[rt][lane * 4 + q];
#pragma unroll
        for (int e = 0; e < 4; ++e) s0[4 * q + e] += x[e];
      }
      // C register i holds row 8 (i / 4) + 4 half + i % 4 of column m: rows increase with i, so
      // the first largest sum is the lowest maximising token.  32-bit compares on the
      // order-preserving encoding (0 = none), then one 64-bit key per lane; scaling by 1 / H
      // (a power of two) keeps the order and the ties.
      uint32_t be = 0u;
      int btok = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tok = tt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        const uint32_t e = tok < T ? enc_f32(s0[i]) : 0u;
        if (e > be) { be = e; btok = tok; }
      }
      if (be != 0u) bk = max_u64(bk, argmax_key(dec_f32(be) * inv_h, btok));
    }
    lds_barrier();                                  // exchange slots free for the next round
  }
  if (hg == 0) {
    bk = max_u64(bk, shfl_xor_u64(bk, 32));
    if (half == 0) sm.best[rt][m] = bk;
  }
  lds_barrier();
  if (tid < PG) {
    uint64_t bb = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) bb = max_u64(bb, sm.best[w][tid]);
    sm.tsel[tid] = (g_cur >= 0 && bb != 0) ? 0x7FFFFFFF - (int)(uint32_t)bb : -1;
  }
  lds_barrier();

  // per document (16 lanes) and head: cosine, key gradient, query-gradient weights
  const int idoc = tid >> 4, sub = tid & 15;
  const int64_t d = grp * PG + idoc;
  const int64_t g = shfl_i64(g_cur, idoc);
  g_cur = g_nxt;
  if (d >= n_docs) return;                         // only in the last group
  const int tsel = sm.tsel[idoc];
  const int64_t bd = (int64_t)b * n_docs + d;
  float4* o = reinterpret_cast<float4*>(dK + bd * P_HD);
  if (tsel < 0) {
    if (sub == 0) {
      sel[2 * bd] = -1;
      sel[2 * bd + 1] = -1;
    }
#pragma unroll
    for (int x = 0; x < P_HD / 4 / 16; ++x) nt_store4(o + sub + 16 * x, 0.f, 0.f, 0.f, 0.f);
    if (sub < H) { ikw[bd * H + sub] = 0.f; wcos[bd * H + sub] = 0.f; }
    return;
  }
  // every load of this phase before its first store (a load issued after a store would wait for it)
  const float w = dDoc[bd] * (1.0f / (float)H);
  const uint16_t* qrow = Qr + ((int64_t)b * T + tsel) * P_HD;
  uint2 qv[H][2];
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int j = 0; j < 2; ++j) qv[h][j] = *reinterpret_cast<const uint2*>(qrow + h * D + 4 * (sub + 16 * j));
  if (sub == 0) {
    sel[2 * bd] = (int32_t)g;
    sel[2 * bd + 1] = tsel;
  }
  const uint16_t* krow = cur + idoc * P_KROW;
  float my_ikw = 0.f, my_wc = 0.f;
#pragma unroll
  for (int h = 0; h < H; ++h) {
    uint2 kv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) kv[j] = *reinterpret_cast<const uint2*>(krow + h * D + 4 * (sub + 16 * j));
    float qq = 0.f, kk = 0.f, qk = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint2 x = qv[h][j], y = kv[j];
      qq = dot2_bf16(x.x, x.x, qq); qq = dot2_bf16(x.y, x.y, qq);
      kk = dot2_bf16(y.x, y.x, kk); kk = dot2_bf16(y.y, y.y, kk);
      qk = dot2_bf16(x.x, y.x, qk); qk = dot2_bf16(x.y, y.y, qk);
    }
    qq = sum16(qq);
    kk = sum16(kk);
    qk = sum16(qk);
    float ca = 0.f, cb = 0.f, ik = 0.f, cs = 0.f;
    if (qq > 0.f && kk > 0.f) {
      const float iq = __builtin_amdgcn_rsqf(qq);   // hardware reciprocal square root (~1 ulp)
      ik = __builtin_amdgcn_rsqf(kk);
      cs = qk * iq * ik;
      ca = w * ik * iq;          // dK = w (q^ - c k^) / |k| = ca q - cb k
      cb = w * ik * ik * cs;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint2 x = qv[h][j], y = kv[j];
      nt_store4(o + h * (D / 4) + sub + 16 * j,
                ca * bf16_lo(x.x) - cb * bf16_lo(y.x), ca * bf16_hi(x.x) - cb * bf16_hi(y.x),
                ca * bf16_lo(x.y) - cb * bf16_lo(y.y), ca * bf16_hi(x.y) - cb * bf16_hi(y.y));
    }
    if (h == sub) { my_ikw = w * ik; my_wc = w * cs; }
  }
  if (sub < H) { ikw[bd * H + sub] = my_ikw; wcos[bd * H + sub] = my_wc; }
}

// Persistent select kernel for H = 8: each workgroup walks groups blockIdx.x,
// blockIdx.x + gridDim.x, ... of one query.  Eight waves: wave (rt, hg) scores
// token tile rt (+4, ...) over heads 4 hg .. 4 hg + 3, and with T <= 128 keeps
// those 32 router rows resident as A operands (128 registers); the two head
// groups add their partial sums through LDS.  While a group is scored, the next
// group's rows and norms and the chunk ids of the group after it are copied into
// LDS; the loop is unrolled by two so every buffer address is static.
template <bool RESIDENT>
__global__ void __launch_bounds__(S8_THREADS)
route_bwd_select8_kernel(const uint16_t* __restrict__ Qr, int T, const uint16_t* __restrict__ Krbar,
                         const float* __restrict__ knorm, int64_t n_chunks, int64_t n_docs,
                         const float* __restrict__ dDoc, const int64_t* __restrict__ gsel, float* __restrict__ dK,
                         int32_t* __restrict__ sel, float* __restrict__ ikw, float* __restrict__ wcos) {
  __shared__ __attribute__((aligned(16))) uint16_t kbuf0[PG * P_KROW];
  __shared__ __attribute__((aligned(16))) uint16_t kbuf1[PG * P_KROW];
  __shared__ __attribute__((aligned(16))) S8Lds sm;
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n_groups = (n_docs + PG - 1) / PG;
  const int64_t stride = gridDim.x;
  int64_t grp = blockIdx.x;
  if (grp >= n_groups) return;
  const int n_tt = (T + 31) / 32;
  bf16x8_t a[4][8];
  if constexpr (RESIDENT) load_rows4(Qr, b, T, (wave & 3) < n_tt ? (wave & 3) : 0, wave >> 2, lane & 31, lane >> 5, a,
                           sm.iq[wave]);
  const int64_t* gs = gsel + (int64_t)b * n_docs;
  const uint32_t voff16 = (uint32_t)lane * 16u, voff4 = (uint32_t)lane * 4u;
  // prologue: this group's chunk ids (lanes 0..31), its copies, and the next group's ids
  int64_t g_cur = -1;
  {
    const int64_t d = grp * PG + (lane & 31);
    if (lane < 32 && d < n_docs) g_cur = gs[d];
  }
  copy_group(Krbar, knorm, n_chunks, g_cur, kbuf0, &sm.ik[0][0][0], wave, lane, voff16);
  copy_ids(gs, n_docs, grp + stride, sm.ids[1], wave, voff4);
  bool first = true;
  while (true) {
    select8_group<RESIDENT>(Qr, b, T, Krbar, knorm, n_chunks, n_docs, dDoc, gs, grp, stride, g_cur, first, kbuf0,
                            kbuf1,
                  &sm.ik[0][0][0], &sm.ik[1][0][0], sm.ids[1], sm.ids[0], a, sm, dK, sel, ikw, wcos, tid,
                  wave, lane, voff16, voff4);
    first = false;
    grp += stride;
    if (grp >= n_groups) break;
    select8_group<RESIDENT>(Qr, b, T, Krbar, knorm, n_chunks, n_docs, dDoc, gs, grp, stride, g_cur, false, kbuf1,
                            kbuf0,
                  &sm.ik[1][0][0], &sm.ik[0][0][0], sm.ids[0], sm.ids[1], a, sm, dK, sel, ikw, wcos, tid,
                  wave, lane, voff16, voff4);
    grp += stride;
    if (grp >= n_groups) break;
  }
  wait_vmem_all();                                 // no copy into LDS outlives the workgroup
}

// Per tile of SORT_TILE documents: how many select each token.
__global__ void __launch_bounds__(256)
route_bwd_hist_kernel(const int32_t* __restrict__ sel, int64_t n_docs, int T, int64_t n_tiles,
                      int32_t* __restrict__ tile_cnt) {
  __shared__ int cnt[MAX_T];
  const int b = blockIdx.y, tid = threadIdx.x;
  const int64_t tile = blockIdx.x;
  for (int t = tid; t < T; t += 256) cnt[t] = 0;
  __syncthreads();
  for (int i = tid; i < SORT_TILE; i += 256) {
    const int64_t d = tile * SORT_TILE + i;
    if (d < n_docs) {
      const int t = sel[((int64_t)b * n_docs + d) * 2 + 1];
      if (t >= 0) atomicAdd(&cnt[t], 1);
    }
  }
  __syncthreads();
  int32_t* out = tile_cnt + ((int64_t)b * n_tiles + tile) * T;
  for (int t = tid; t < T; t += 256) out[t] = cnt[t];
}

// One workgroup per query: each token's segment in the sorted order (seg), its
// pieces (pstart), the piece -> token table, and, in place of the tile counts,
// each tile's offset inside the token's segment.
__global__ void __launch_bounds__(1024)
route_bwd_scan_kernel(int32_t* __restrict__ tile_cnt, int64_t n_tiles, int T, int64_t max_pieces,
                      int32_t* __restrict__ seg, int32_t* __restrict__ pstart, int4* __restrict__ pdesc) {
  constexpr int U = 16;
  __shared__ int64_t s_a[16], s_b[16];
  __shared__ int64_t carry_a, carry_b;
  const int b = blockIdx.x, tid = threadIdx.x;
  int32_t* tc = tile_cnt + (int64_t)b * n_tiles * T;
  int32_t* sg = seg + (int64_t)b * (T + 1);
  int32_t* ps = pstart + (int64_t)b * (T + 1);
  int4* pd = pdesc + (int64_t)b * max_pieces;
  if (tid == 0) { carry_a = 0; carry_b = 0; }
  __syncthreads();
  for (int t0 = 0; t0 < T; t0 += 1024) {
    const int t = t0 + tid;
    int64_t tot = 0;
    if (t < T) {
      int64_t k0 = 0;
      for (; k0 + U <= n_tiles; k0 += U) {
        int32_t c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) c[u] = tc[(k0 + u) * T + t];
#pragma unroll
        for (int u = 0; u < U; ++u) { tc[(k0 + u) * T + t] = (int32_t)tot; tot += c[u]; }
      }
      for (; k0 < n_tiles; ++k0) {
        const int32_t c = tc[k0 * T + t];
        tc[k0 * T + t] = (int32_t)tot;
        tot += c;
      }
    }
    const int64_t np = (tot + PIECE - 1) / PIECE;
    int64_t a = tot, p = np;
    block_scan2(a, p, s_a, s_b);
    const int64_t ca = carry_a, cb = carry_b;
    if (t < T) {
      const int64_t p0 = cb + p - np;
      sg[t] = (int32_t)(ca + a - tot);
      ps[t] = (int32_t)p0;
      const int64_t s0 = ca + a - tot;
      for (int64_t j = 0; j < np; ++j) {
        const int64_t left = tot - j * PIECE;
        pd[p0 + j] = make_int4(t, (int)(s0 + j * PIECE), (int)(left < PIECE ? left : PIECE), 0);
      }
    }
    __syncthreads();
    if (tid == 1023) { carry_a = ca + a; carry_b = cb + p; }
    __syncthreads();
  }
  if (tid == 0) { sg[T] = (int32_t)carry_a; ps[T] = (int32_t)carry_b; }
  for (int64_t j = carry_b + tid; j < max_pieces; j += 1024) pd[j] = make_int4(0, 0, 0, 0);   // unused: empty
}

// Stable scatter: document d goes to its token's segment after every earlier
// document with the same token.
__global__ void __launch_bounds__(256)
route_bwd_scatter_kernel(const int32_t* __restrict__ sel, int64_t n_docs, int T, int64_t n_tiles,
                         const int32_t* __restrict__ tile_cnt, const int32_t* __restrict__ seg,
                         int32_t* __restrict__ order, int64_t* __restrict__ ordg) {
  __shared__ int base[MAX_T];
  __shared__ __attribute__((aligned(16))) int t_s[256];
  const int b = blockIdx.y, tid = threadIdx.x, wave = tid >> 6;
  const int64_t tile = blockIdx.x;
  const int32_t* tc = tile_cnt + ((int64_t)b * n_tiles + tile) * T;
  const int32_t* sg = seg + (int64_t)b * (T + 1);
  for (int t = tid; t < T; t += 256) base[t] = sg[t] + tc[t];
  __syncthreads();
  for (int sb = 0; sb < SORT_TILE; sb += 256) {
    if (tile * SORT_TILE + sb >= n_docs) break;
    const int64_t d = tile * SORT_TILE + sb + tid;
    int2 gt = make_int2(-1, -1);
    if (d < n_docs) gt = *reinterpret_cast<const int2*>(sel + ((int64_t)b * n_docs + d) * 2);
    const int t = gt.y;
    t_s[tid] = t;
    __syncthreads();
    // rank among the earlier documents of this block with the same token
    int rank = 0;
    const int n4 = (wave + 1) * 16;
#pragma unroll 4
    for (int j4 = 0; j4 < n4; ++j4) {
      const int4 v = *reinterpret_cast<const int4*>(&t_s[4 * j4]);
      const int j = 4 * j4;
      rank += (j < tid && v.x == t) + (j + 1 < tid && v.y == t) + (j + 2 < tid && v.z == t) +
              (j + 3 < tid && v.w == t);
    }
    if (t >= 0) {
      const int64_t pos = (int64_t)b * n_docs + base[t] + rank;
      order[pos] = (int32_t)d;
      ordg[pos] = gt.x;
    }
    __syncthreads();
    if (t >= 0) atomicAdd(&base[t], 1);
    __syncthreads();
  }
}

// One piece of one token's list: sum over its documents of (w/|k|) k and w c.
// Thread x owns 8 dims of the H*D row and every RG-th document of the piece; the
// RG row groups are then added in order.
template <int H>
__global__ void __launch_bounds__(256)
route_bwd_piece_kernel(const uint16_t* __restrict__ Krbar, int64_t n_docs, const float* __restrict__ ikw,
                       const float* __restrict__ wcos, const int32_t* __restrict__ order,
                       const int64_t* __restrict__ ordg, const int4* __restrict__ pdesc, int64_t max_pieces,
                       float* __restrict__ partial, float* __restrict__ partial_c) {
  constexpr int HD = H * D, TPR = HD / 8, RG = 256 / TPR;
  __shared__ int64_t g_s[PIECE], bd_s[PIECE];
  __shared__ __attribute__((aligned(16))) float red[RG][HD];
  __shared__ float red_c[RG][H];
  const int b = blockIdx.y, tid = threadIdx.x;
  const int64_t p = blockIdx.x;
  const int4 pd = pdesc[(int64_t)b * max_pieces + p];       // (token, first position, count)
  const int n = pd.z;
  if (n == 0) return;
  if (tid < n) {
    const int64_t pos = (int64_t)b * n_docs + pd.y + tid;
    bd_s[tid] = (int64_t)b * n_docs + order[pos];
    g_s[tid] = ordg[pos];
  }
  __syncthreads();
  const int rg = tid / TPR, e0 = 8 * (tid % TPR), h = e0 / D;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float cs = 0.f;
  for (int j0 = rg; j0 < n; j0 += RG * PIECE_UNROLL) {
    uint4 kv[PIECE_UNROLL];
    float iw[PIECE_UNROLL], wc[PIECE_UNROLL];
#pragma unroll
    for (int u = 0; u < PIECE_UNROLL; ++u) {
      const int j = j0 + u * RG;
      if (j < n) {
        const int64_t bd = bd_s[j];
        kv[u] = *reinterpret_cast<const uint4*>(Krbar + g_s[j] * HD + e0);
        iw[u] = ikw[bd * H + h];
        wc[u] = wcos[bd * H + h];
      }
    }
#pragma unroll
    for (int u = 0; u < PIECE_UNROLL; ++u) {
      if (j0 + u * RG < n) {
        const uint32_t x[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += iw[u] * bf16_lo(x[e]);
          acc[2 * e + 1] += iw[u] * bf16_hi(x[e]);
        }
        cs += wc[u];
      }
    }
  }
  *reinterpret_cast<float4*>(&red[rg][e0]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(&red[rg][e0 + 4]) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  if ((e0 & (D - 1)) == 0) red_c[rg][h] = cs;
  __syncthreads();
  if (rg != 0) return;
  for (int r = 1; r < RG; ++r) {
    const float4 x0 = *reinterpret_cast<const float4*>(&red[r][e0]);
    const float4 x1 = *reinterpret_cast<const float4*>(&red[r][e0 + 4]);
    acc[0] += x0.x; acc[1] += x0.y; acc[2] += x0.z; acc[3] += x0.w;
    acc[4] += x1.x; acc[5] += x1.y; acc[6] += x1.z; acc[7] += x1.w;
    cs += red_c[r][h];
  }
  float* o = partial + ((int64_t)b * max_pieces + p) * HD + e0;
  *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  if ((e0 & (D - 1)) == 0) partial_c[((int64_t)b * max_pieces + p) * H + h] = cs;
}

// One token: its pieces in order, then dq = (A - q^ C) / |q| per head.
__global__ void __launch_bounds__(256)
route_bwd_final_kernel(const uint16_t* __restrict__ Qr, int T, int H, const int32_t* __restrict__ pstart,
                       int64_t max_pieces, const float* __restrict__ partial, const float* __restrict__ partial_c,
                       float* __restrict__ dQ) {
  constexpr int U = 8;
  const int t = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int HD = H * D, e0 = 4 * tid, h = e0 / D;
  if (e0 >= HD) return;
  const int32_t* ps = pstart + (int64_t)b * (T + 1);
  const int64_t p1 = ps[t + 1];
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float cs = 0.f;
  for (int64_t p0 = ps[t]; p0 < p1; p0 += U) {
    float4 v[U];
    float c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (p0 + u < p1) {
        v[u] = *reinterpret_cast<const float4*>(partial + ((int64_t)b * max_pieces + p0 + u) * HD + e0);
        c[u] = partial_c[((int64_t)b * max_pieces + p0 + u) * H + h];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (p0 + u < p1) {
        acc[0] += v[u].x; acc[1] += v[u].y; acc[2] += v[u].z; acc[3] += v[u].w;
        cs += c[u];
      }
    }
  }
  const uint2 qv = *reinterpret_cast<const uint2*>(Qr + ((int64_t)b * T + t) * HD + e0);
  const float q[4] = {bf16_lo(qv.x), bf16_hi(qv.x), bf16_lo(qv.y), bf16_hi(qv.y)};
  float ss = dot2_bf16(qv.x, qv.x, 0.f);
  ss = dot2_bf16(qv.y, qv.y, ss);
#pragma unroll
  for (int s = 1; s < 32; s <<= 1) ss += __shfl_xor(ss, s);   // the 32 threads of head h
  const float iq = inv_norm(ss);
  *reinterpret_cast<float4*>(dQ + ((int64_t)b * T + t) * HD + e0) =
      make_float4(iq * (acc[0] - iq * q[0] * cs), iq * (acc[1] - iq * q[1] * cs), iq * (acc[2] - iq * q[2] * cs),
                  iq * (acc[3] - iq * q[3] * cs));
}

struct BwdLayout {
  int64_t n_tiles, max_pieces;
  size_t ikw, wcos, tile_cnt, seg, pstart, pdesc, order, ordg, partial, partial_c, gsel, total;
};

BwdLayout bwd_layout(int B, int T, int H, int64_t n_docs) {
  BwdLayout L;
  size_t o = 0;
  auto take = [&o](size_t bytes) {
    const size_t at = o;
    o += (bytes + 255) & ~(size_t)255;
    return at;
  };
  const size_t Bz = (size_t)B;
  L.n_tiles = (n_docs + SORT_TILE - 1) / SORT_TILE;
  L.max_pieces = (n_docs + PIECE - 1) / PIECE + T;
  L.ikw = take(Bz * n_docs * H * 4);
  L.wcos = take(Bz * n_docs * H * 4);
  L.tile_cnt = take(Bz * L.n_tiles * T * 4);
  L.seg = take(Bz * (T + 1) * 4);
  L.pstart = take(Bz * (T + 1) * 4);
  L.pdesc = take(Bz * L.max_pieces * 16);
  L.order = take(Bz * n_docs * 4);
  L.ordg = take(Bz * n_docs * 8);
  L.partial = take(Bz * L.max_pieces * H * D * 4);
  L.partial_c = take(Bz * L.max_pieces * H * 4);
  L.gsel = take(H == 8 ? Bz * n_docs * 8 : 0);
  L.total = o;
  return L;
}

struct BwdArgs {
  const uint16_t* Qr; int B, T; const uint16_t* Krbar; const float* knorm; int64_t n_chunks;
  const int64_t* off; int64_t n_docs; const uint8_t* exclude; const float* chunk_scores; const float* dDoc;
  float* dQ; float* dK; int32_t* sel;
};

template <int H>
int launch_bwd_h(const BwdArgs& A, const BwdLayout& L, uint8_t* ws, hipStream_t stream) {
  float* ikw = reinterpret_cast<float*>(ws + L.ikw);
  float* wcos = reinterpret_cast<float*>(ws + L.wcos);
  int32_t* tile_cnt = reinterpret_cast<int32_t*>(ws + L.tile_cnt);
  int32_t* seg = reinterpret_cast<int32_t*>(ws + L.seg);
  int32_t* pstart = reinterpret_cast<int32_t*>(ws + L.pstart);
  int4* pdesc = reinterpret_cast<int4*>(ws + L.pdesc);
  int32_t* order = reinterpret_cast<int32_t*>(ws + L.order);
  int64_t* ordg = reinterpret_cast<int64_t*>(ws + L.ordg);
  float* partial = reinterpret_cast<float*>(ws + L.partial);
  float* partial_c = reinterpret_cast<float*>(ws + L.partial_c);
  const int B = A.B, T = A.T;
  const int64_t n_docs = A.n_docs;
  if constexpr (H == 8) {
    int64_t* gsel = reinterpret_cast<int64_t*>(ws + L.gsel);
    hipLaunchKernelGGL(route_bwd_pick_kernel, dim3((unsigned)((n_docs * LPD + 255) / 256), (unsigned)B), dim3(256), 0,
                       stream, A.off, n_docs, A.n_chunks, A.exclude, A.chunk_scores, A.dDoc, gsel);
    MSA_CHECK_LAUNCH();
    // one persistent workgroup per CU (its LDS holds two groups of rows)
    const int64_t n_groups = (n_docs + PG - 1) / PG;
    int64_t per_b = (SELECT8_WORKGROUPS + B - 1) / B;
    per_b = per_b < n_groups ? per_b : n_groups;
    if (T <= 128)
      hipLaunchKernelGGL(route_bwd_select8_kernel<true>, dim3((unsigned)per_b, (unsigned)B), dim3(S8_THREADS), 0,
                         stream, A.Qr, T, A.Krbar, A.knorm, A.n_chunks, n_docs, A.dDoc, gsel, A.dK, A.sel,
                         ikw, wcos);
    else
      hipLaunchKernelGGL(route_bwd_select8_kernel<false>, dim3((unsigned)per_b, (unsigned)B), dim3(S8_THREADS), 0,
                         stream, A.Qr, T, A.Krbar, A.knorm, A.n_chunks, n_docs, A.dDoc, gsel, A.dK, A.sel,
                         ikw, wcos);
    MSA_CHECK_LAUNCH();
  } else {
    hipLaunchKernelGGL(route_bwd_select_kernel<H>, dim3((unsigned)((n_docs + SEL_DOCS - 1) / SEL_DOCS), (unsigned)B),
                       dim3(SEL_THREADS), 0, stream, A.Qr, T, A.Krbar, A.knorm, A.off, n_docs, A.n_chunks, A.exclude,
                       A.chunk_scores, A.dDoc, A.dK, A.sel, ikw, wcos);
    MSA_CHECK_LAUNCH();
  }
  const dim3 gt((unsigned)L.n_tiles, (unsigned)B);
  hipLaunchKernelGGL(route_bwd_hist_kernel, gt, dim3(256), 0, stream, A.sel, n_docs, T, L.n_tiles, tile_cnt);
  MSA_CHECK_LAUNCH();
  hipLaunchKernelGGL(route_bwd_scan_kernel, dim3((unsigned)B), dim3(1024), 0, stream, tile_cnt, L.n_tiles, T,
                     L.max_pieces, seg, pstart, pdesc);
  MSA_CHECK_LAUNCH();
  hipLaunchKernelGGL(route_bwd_scatter_kernel, gt, dim3(256), 0, stream, A.sel, n_docs, T, L.n_tiles, tile_cnt, seg,
                     order, ordg);
  MSA_CHECK_LAUNCH();
  hipLaunchKernelGGL(route_bwd_piece_kernel<H>, dim3((unsigned)L.max_pieces, (unsigned)B), dim3(256), 0, stream,
                     A.Krbar, n_docs, ikw, wcos, order, ordg, pdesc, L.max_pieces, partial, partial_c);
  MSA_CHECK_LAUNCH();
  hipLaunchKernelGGL(route_bwd_final_kernel, dim3((unsigned)T, (unsigned)B), dim3(256), 0, stream, A.Qr, T, H,
                     pstart, L.max_pieces, partial, partial_c, A.dQ);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

}  // namespace

size_t route_bwd_workspace(int B, int T, int H, int64_t n_docs) { return bwd_layout(B, T, H, n_docs).total; }

int launch_route_bwd(const uint16_t* Qr, int B, int T, int H, const uint16_t* Krbar, const float* inv_norm_k,
                     int64_t n_chunks, const int64_t* off, int64_t n_docs, const uint8_t* exclude,
                     const float* chunk_scores, const float* dDoc, float* dQ, float* dK, int32_t* sel,
                     void* workspace, hipStream_t stream) {
  const BwdLayout L = bwd_layout(B, T, H, n_docs);
  const BwdArgs A{Qr, B, T, Krbar, inv_norm_k, n_chunks, off, n_docs, exclude, chunk_scores, dDoc, dQ, dK, sel};
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  switch (H) {
    case 1: return launch_bwd_h<1>(A, L, ws, stream);
    case 2: return launch_bwd_h<2>(A, L, ws, stream);
    case 4: return launch_bwd_h<4>(A, L, ws, stream);
    case 8: return launch_bwd_h<8>(A, L, ws, stream);
    default: set_error("route backward: H=%d unsupported", H); return MSA_ERR_UNSUPPORTED;
  }
}

}  // namespace msa
