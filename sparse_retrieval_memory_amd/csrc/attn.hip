// Sparse attention over [pooled memory ++ causal local KV] (medium write-up
// sec. 2 and b-lab.team summary sec. 1: the selected documents' compressed
// K/V are concatenated with the query's local K/V for autoregressive
// decoding; b-lab.team sec. 1, Global RoPE: the query's start index is offset
// by k, the number of retrieved blocks).
//
// Flash-style on the matrix cores.  One workgroup owns 32 query rows of one
// q-head; its 8 waves (two per SIMD) take runs of consecutive tiles of 32 keys
// (memory entries first, then local keys up to the causal limit of the last
// row) and keep a running max, sum and output per row; the waves' partial
// results are merged at the end.  Per key tile, a wave computes S^T = K Q^T
// (keys x rows) with v_mfma_f32_32x32x16_bf16, so every lane holds one query
// row's scores, and the softmax statistics of a row live in one lane pair.
// O^T += V^T P^T then uses the same layout: V is copied to LDS by LDS DMA and
// read back transposed by ds_read_b64_tr_b16.
//
// Precision: the operands of both products are split into bf16 hi + lo parts
// (q = qh + ql with |ql| <= 2^-9 |q|), so with fp32 accumulation the scores
// and weighted sums keep ~2^-16 relative accuracy instead of bf16's 2^-8.
// Memory keys and V are bf16 already (no lo part); rotated local keys and
// queries, and the probabilities, are split.  RoPE angles are reduced in fp64
// (position x frequency in revolutions) and evaluated in fp32; up to 128 local
// positions the workgroup first builds a cos/sin table in LDS (an exact value
// every 32 positions, then 8-position and one-position rotations, at most 10
// from an exact value) that the query rows and local keys read.  Scores are
// pre-scaled by scale * log2(e) so the exponentials are exp2.
#include "msa_internal.h"
#include "attn_split.h"

#include <math.h>

namespace msa {
namespace {

constexpr int D = 128;
constexpr int RT = 32;          // query rows per workgroup (MFMA N)
constexpr int KT = 32;          // keys per tile (MFMA M)
constexpr int NWAVE = 8;        // two waves per SIMD
constexpr int THREADS = 64 * NWAVE;
constexpr int V_ROW = D * 2;        // bytes of one key's V row in a wave's LDS buffer
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

struct bf16pair {
  bf16x8_t hi, lo;
};

__device__ __forceinline__ uint32_t pack2(uint32_t a, uint32_t b) { return a | (b << 16); }

// x -> (bf16 hi, bf16 lo) with hi = RNE(x), lo = RNE(x - hi); 8 values.
__device__ __forceinline__ bf16pair split8(const float (&x)[8]) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = cvt2_bf16(x[2 * j], x[2 * j + 1]);
    l[j] = cvt2_bf16(x[2 * j] - bf16_lo(h[j]), x[2 * j + 1] - bf16_hi(h[j]));
  }
  bf16pair r;
  r.hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  r.lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
  return r;
}

__device__ __forceinline__ void unpack8(uint4 v, float (&x)[8]) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// Rotate the pairs (i, i + 64) held by one lane: lo[j] = dims 16 ks + 8 hf + j
// (ks < 4), hi[j] = the same dims + 64.
__device__ __forceinline__ void rotate_pairs(float (&lo)[8], float (&hi)[8], int pos, const double* rev, int d0) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float c, s;
    rope_cs(pos, rev[d0 + j], &c, &s);
    const float x1 = lo[j], x2 = hi[j];
    lo[j] = x1 * c - x2 * s;
    hi[j] = x2 * c + x1 * s;
  }
}

// The same rotation with cos/sin read from a table: cs[p][i] = (cos, sin) of
// position base + p at frequency i (the table of the workgroup's positions).
__device__ __forceinline__ void rotate_pairs_tab(float (&lo)[8], float (&hi)[8], const float2* cs_row, int d0) {
  const float4* t = reinterpret_cast<const float4*>(cs_row + d0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = t[q];
    const float c0 = v.x, s0 = v.y, c1 = v.z, s1 = v.w;
    float x1 = lo[2 * q], x2 = hi[2 * q];
    lo[2 * q] = x1 * c0 - x2 * s0;
    hi[2 * q] = x2 * c0 + x1 * s0;
    x1 = lo[2 * q + 1]; x2 = hi[2 * q + 1];
    lo[2 * q + 1] = x1 * c1 - x2 * s1;
    hi[2 * q + 1] = x2 * c1 + x1 * s1;
  }
}

constexpr int TAB_POS = 128;    // positions the LDS cos/sin table covers (local keys and queries)
// Which keys a launch covers and what it writes:
//   FULL   memory entries ++ local keys; O (and optionally the log-sum-exp)
//   LOCAL  local keys only; the unnormalised partial sum, its row max and sum (PO, PML)
//   MEMORY memory entries only, merged with a LOCAL partial; O (and optionally the log-sum-exp)
// LOCAL needs nothing retrieved, so it can run while the memory is still being selected and
// assembled; LOCAL + MEMORY give the same O as FULL up to the order of the sums.
constexpr int MODE_FULL = 0, MODE_LOCAL = 1, MODE_MEMORY = 2;
constexpr int TAB_SEG = 32;     // positions one thread steps through from an exact start
constexpr int PART_STRIDE = D + 4;   // floats per (wave, row) in the merge area: 16-byte rows skewed by 4 banks

// RoPE constants computed on the host in fp64 and passed with the launch:
// rev[i] = theta_i / (2 pi); start[sg][i] = (cos, sin) at position rope_offset +
// TAB_SEG * sg; step[i], step8[i] = (cos, sin) of one and of eight positions.
struct RopeTables {
  double rev[D / 2];
  float2 start[TAB_POS / TAB_SEG][D / 2];
  float2 step[D / 2];
  float2 step8[D / 2];
};

// One table thread's share: positions p0 .. p0 + TAB_SEG - 1 (below n_pos) at frequency i, as 4
// interleaved runs of 8.  From the exact (cos, sin) at p0 the runs' starts follow by exact 8-position
// rotations and each run by exact one-position rotations, so every entry is at most 10 rotations
// from an exact value (error ~1e-6).
__device__ __forceinline__ void fill_cs_segment(float2 (*cs_tab)[D / 2 + 2], int i, int p0, int n_pos, float2 st,
                                                float2 d1, float2 d8) {
  static_assert(TAB_SEG == 4 * 8, "four runs of eight positions per segment");
  float c[4], s_[4];
  c[0] = st.x;
  s_[0] = st.y;
#pragma unroll
  for (int m = 1; m < 4; ++m) {
    c[m] = c[m - 1] * d8.x - s_[m - 1] * d8.y;
    s_[m] = s_[m - 1] * d8.x + c[m - 1] * d8.y;
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int p = p0 + 8 * m + u;
      if (p < n_pos) cs_tab[p][i] = make_float2(c[m], s_[m]);
      const float cn = c[m] * d1.x - s_[m] * d1.y;
      s_[m] = s_[m] * d1.x + c[m] * d1.y;
      c[m] = cn;
    }
  }
}

__global__ void __launch_bounds__(THREADS, 1)
attn_mfma_kernel(const uint16_t* __restrict__ Q, int Tq, int Hq, const uint16_t* __restrict__ Kloc,
                 const uint16_t* __restrict__ Vloc, int Tl, int Hkv, const uint16_t* __restrict__ Kmem,
                 const uint16_t* __restrict__ Vmem, int64_t mstride, int Mmax, const int32_t* __restrict__ mem_len,
                 int rope_offset, const RopeTables tabs, float scale_log2e, float* __restrict__ O,
                 float* __restrict__ LSE, int mode, float* __restrict__ PO, float* __restrict__ PML) {
  __shared__ double rev[D / 2];
  // LDS: first cos/sin of positions rope_offset + p (p < n_local <= TAB_POS), frequency i: every
  // query row and local key of this workgroup sits at such a position.  Rows are padded by 16
  // bytes: the 32 lanes of a rotation read 32 consecutive positions at one frequency, which with
  // 512-byte rows would all fall in the same four banks.  Then, per wave, V of its current tile
  // (KT rows of V_ROW bytes).  The merge's partial outputs overwrite both once every tile is done.
  constexpr int TAB_FLOATS = TAB_POS * (D / 2 + 2) * 2;
  constexpr int V_FLOATS = NWAVE * KT * V_ROW / 4;
  constexpr int PART_FLOATS = NWAVE * RT * PART_STRIDE;
  __shared__ __attribute__((aligned(16))) float lds[TAB_FLOATS + V_FLOATS > PART_FLOATS ? TAB_FLOATS + V_FLOATS
                                                                                       : PART_FLOATS];
  float2 (*cs_tab)[D / 2 + 2] = reinterpret_cast<float2 (*)[D / 2 + 2]>(lds);
  __shared__ float m_sh[NWAVE][RT], l_sh[NWAVE][RT];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, hf = lane >> 5;
  const int r0 = blockIdx.x * RT;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int g = h / (Hq / Hkv);
  int last = r0 + RT - 1;
  if (last > Tq - 1) last = Tq - 1;
  const int n_pos = (Tl - Tq) + last + 1;          // positions of this tile's rows and their local keys
  const int n_local = mode == MODE_MEMORY ? 0 : n_pos;

  // Loads in the order their data is needed (vector loads complete in order): the table's
  // constants, then the query rows and the memory length, whose latency overlaps the table set-up.
  const bool use_tab = n_pos <= TAB_POS;
  const int ti = tid & (D / 2 - 1), tsg = tid / (D / 2);
  static_assert(THREADS >= TAB_POS / TAB_SEG * (D / 2), "one segment per thread covers the table");
  const bool tab_thread = use_tab && tid < TAB_POS / TAB_SEG * (D / 2) && tsg * TAB_SEG < n_pos;
  float2 t_st = make_float2(0.f, 0.f), t_d1 = t_st, t_d8 = t_st;
  if (tab_thread) {
    t_st = tabs.start[tsg][ti];
    t_d1 = tabs.step[ti];
    t_d8 = tabs.step8[ti];
  }
  const int row = r0 + col;
  uint4 qraw[8];
  {
    // rows past the end read the last row (unconditional loads keep the waits' counts exact);
    // their values are replaced by zeros below
    const uint16_t* q = Q + (((int64_t)b * Tq + (row < Tq ? row : Tq - 1)) * Hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qraw[ks] = *reinterpret_cast<const uint4*>(q + 16 * ks + 8 * hf);
      qraw[ks + 4] = *reinterpret_cast<const uint4*>(q + 64 + 16 * ks + 8 * hf);
    }
  }
  const int m_in = mode == MODE_LOCAL ? 0 : mem_len[b];

  if (!use_tab && tid < D / 2) rev[tid] = tabs.rev[tid];
  // Table for n_local <= TAB_POS: thread (frequency ti, segment tsg) fills the segment's positions.
  if (tab_thread) fill_cs_segment(cs_tab, ti, tsg * TAB_SEG, n_pos, t_st, t_d1, t_d8);
  __syncthreads();

  const int M = m_in < 0 ? 0 : (m_in > Mmax ? Mmax : m_in);
  const int n_keys = M + n_local;
  const int n_tiles = (n_keys + KT - 1) / KT;

  // Row of key j (memory entry j < M, else local key j - M) of this workgroup's kv head, with the
  // choice made on offsets (one select instead of two address paths)
  const int64_t mem_base = (int64_t)b * Mmax * mstride + (int64_t)g * D;
  const int64_t loc_base = ((int64_t)b * Tl - M) * Hkv * D + (int64_t)g * D;
  const int64_t loc_stride = (int64_t)Hkv * D;
  auto key_row = [&](const uint16_t* mem, const uint16_t* loc, int j) -> const uint16_t* {
    const bool in_mem = j < M;
    const int64_t off = in_mem ? mem_base + (int64_t)j * mstride : loc_base + (int64_t)j * loc_stride;
    return (in_mem ? mem : loc) + off;
  };
  // Raw K of key tile t for this lane (key k0 + col) in registers: dims 16 (ks % 4) + 64 (ks / 4) +
  // 8 hf + e (the A-operand order).  Keys past the end read the tile's first key (unconditional
  // loads keep the waits' counts exact); their scores are masked.
  auto load_k = [&](int t, uint4 (&kr)[8], bool& local) {
    const int j0 = t * KT + col;
    const int j = j0 < n_keys ? j0 : t * KT;
    local = j0 < n_keys && j0 >= M;
    const uint16_t* kp = key_row(Kmem, Kloc, j);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      kr[ks] = *reinterpret_cast<const uint4*>(kp + 16 * (ks & 3) + 64 * (ks >> 2) + 8 * hf);
  };
  // V of key tile t into this wave's LDS buffer by 8 LDS-DMA copies of 1 KB: copy n fills rows
  // 4n .. 4n + 3; lane l fills row 4n + l / 16, 16-byte slot l % 16, which holds dims 8 p .. 8 p + 7
  // of the row's key with p = slot ^ 4 (row % 4) (the swizzle makes the transposing reads below
  // conflict-free).  Keys past the end copy the tile's first key: their probabilities are zero.
  uint8_t* const vbuf = reinterpret_cast<uint8_t*>(lds + TAB_FLOATS) + wave * KT * V_ROW;
  const int64_t v_piece = 8 * ((lane & 15) ^ ((lane >> 4) << 2));   // this lane's 16-byte slot's dims
  auto load_v = [&](int t) {
    // row 4n + r4 of the tile: offsets advance by 4 rows per copy in both address ranges
    const int j0 = t * KT + (lane >> 4);
    int64_t om = mem_base + (int64_t)j0 * mstride + v_piece;
    int64_t ol = loc_base + (int64_t)j0 * loc_stride + v_piece;
    // the tile's first key, read in place of keys past the end
    const bool first_mem = t * KT < M;
    const int64_t of = (first_mem ? mem_base + (int64_t)(t * KT) * mstride
                                  : loc_base + (int64_t)(t * KT) * loc_stride) + v_piece;
#pragma unroll
    for (int n = 0; n < KT / 4; ++n) {
      const int j = j0 + 4 * n;
      const bool in_mem = j < M, valid = j < n_keys;
      const bool use_mem = valid ? in_mem : first_mem;
      const int64_t off = valid ? (in_mem ? om : ol) : of;
      dma16((use_mem ? Vmem : Vloc) + off, vbuf + 4 * V_ROW * n);
      om += 4 * mstride;
      ol += 4 * loc_stride;
    }
  };

  // wave w takes a run of consecutive tiles; the first n_tiles % NWAVE waves take one more, so the
  // longer runs start with memory tiles, which cost less than local ones (no rotation or split)
  const int per = n_tiles / NWAVE, extra = n_tiles % NWAVE;
  const int t_begin = wave * per + (wave < extra ? wave : extra);
  const int t_end = t_begin + per + (wave < extra ? 1 : 0);
  // The first tile's V copies overlap the query set-up.  The query rows have arrived long since;
  // waiting for them here keeps the wait before their use from also covering these copies.
  __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0)
  if (t_begin < t_end) load_v(t_begin);

  // ---- Q^T as the B operand: lane (col, hf) holds query row r0 + col, dims 16 ks + 8 hf + j
  bf16x8_t qh[8], ql[8];
  {
    float lo[4][8], hi[4][8];
    if (row < Tq) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        unpack8(qraw[ks], lo[ks]);
        unpack8(qraw[ks + 4], hi[ks]);
      }
      const int p = (Tl - Tq) + row;
      if (use_tab) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) rotate_pairs_tab(lo[ks], hi[ks], cs_tab[p], 16 * ks + 8 * hf);
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) rotate_pairs(lo[ks], hi[ks], rope_offset + p, rev, 16 * ks + 8 * hf);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) { lo[ks][j] = 0.f; hi[ks][j] = 0.f; }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int j = 0; j < 8; ++j) { lo[ks][j] *= scale_log2e; hi[ks][j] *= scale_log2e; }
      const bf16pair a = split8(lo[ks]), c = split8(hi[ks]);
      qh[ks] = a.hi; ql[ks] = a.lo;
      qh[ks + 4] = c.hi; ql[ks + 4] = c.lo;
    }
  }

  // running state of this lane's query row (both lanes of a pair keep identical copies)
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t oacc[4];   // O^T: dim tile dt, rows = dims 32 dt + 8 (i/4) + 4 hf + i % 4, column = query row
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;

  const int qrow = r0 + col;
  const int lim = (Tl - Tq) + qrow;      // last visible local key of this row

  for (int t = t_begin; t < t_end; ++t) {
    const int k0 = t * KT;
    const int j = k0 + col;
    uint4 kc[8];
    bool local;
    load_k(t, kc, local);
    if (t != t_begin) load_v(t);
    f32x16_t s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    const bool tile_local = __builtin_amdgcn_readfirstlane((int)(k0 + KT > M && M < n_keys)) != 0;
    if (!tile_local) {
      // memory keys only: exact bf16 operands, Q split in two (two accumulation chains)
      f32x16_t s2;
#pragma unroll
      for (int i = 0; i < 16; ++i) s2[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, kc[ks]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qh[ks], s, 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, ql[ks], s2, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] += s2[i];
    } else {
      // local keys (or a tile holding both kinds): rotate in fp32, split in two; a dim block
      // ks < 4 and its RoPE partners ks + 4 at a time, so few unpacked values are live
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float lo[8], hi[8];
        unpack8(kc[ks], lo);
        unpack8(kc[ks + 4], hi);
        if (local) {
          if (use_tab) rotate_pairs_tab(lo, hi, cs_tab[j - M], 16 * ks + 8 * hf);
          else rotate_pairs(lo, hi, rope_offset + (j - M), rev, 16 * ks + 8 * hf);
        }
        const bf16pair ka = split8(lo), kb = split8(hi);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka.hi, qh[ks], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka.hi, ql[ks], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka.lo, qh[ks], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb.hi, qh[ks + 4], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb.hi, ql[ks + 4], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb.lo, qh[ks + 4], s, 0, 0, 0);
      }
    }

    // ---- mask and online softmax for this lane's row (keys 8 (i/4) + 4 hf + i % 4 of the tile)
    float tmax = -INFINITY;
    // every (row, key) of the tile visible: all rows exist and the last key is within the
    // first row's causal limit (memory keys always are)
    const bool all_vis = r0 + RT <= Tq && k0 + KT <= n_keys && k0 + KT - 1 - M <= (Tl - Tq) + r0;
    if (all_vis) {
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * hf + (i & 3);
        bool vis = key < n_keys && qrow < Tq;
        if (key >= M) vis = vis && (key - M) <= lim;
        s[i] = vis ? s[i] : -INFINITY;
        tmax = fmaxf(tmax, s[i]);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float p[16], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = (m_new == -INFINITY) ? 0.f : exp2f(s[i] - m_new);
      psum += p[i];
    }
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;

    // ---- P^T as the B operand (keys 16 st + 8 hf + e of this lane's row): swap halves with the partner
    float send[8], recv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      send[e] = hf == 0 ? p[4 + e] : p[e];
      send[4 + e] = hf == 0 ? p[12 + e] : p[8 + e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) recv[e] = __shfl_xor(send[e], 32);
    float pb[2][8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pb[0][e] = hf == 0 ? p[e] : recv[e];
      pb[0][4 + e] = hf == 0 ? recv[e] : p[4 + e];
      pb[1][e] = hf == 0 ? p[8 + e] : recv[4 + e];
      pb[1][4 + e] = hf == 0 ? recv[4 + e] : p[12 + e];
    }
    const bf16pair p0 = split8(pb[0]), p1 = split8(pb[1]);

    // ---- O^T += V^T P^T: A = V^T (32 dims x 16 keys) by transposing LDS reads.  In each 16-lane
    // group a read hands lane i element i % 4 of the 8-byte piece that lane 4 r + i / 4 addresses,
    // as its element r; so lane (col, hf) receives dim 32 dt + col of keys 16 st + 8 hf + 4 h + r when
    // lane 4 r + c of its group addresses dims 32 dt + 16 (col / 16) + 4 c .. + 3 of that key's row.
    const int gi = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        i16x4_t part[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 16 * st + 8 * hf + 4 * h + (gi >> 2);
          const int p = 4 * dt + 2 * ((lane >> 4) & 1) + ((gi & 3) >> 1);    // logical 16-byte slot
          const int off = row * V_ROW + ((p ^ ((row & 3) << 2)) << 4) + ((gi & 1) << 3);
          part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vbuf + off));
        }
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, st == 0 ? p0.hi : p1.hi, oacc[dt], 0, 0, 0);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, st == 0 ? p0.lo : p1.lo, oacc[dt], 0, 0, 0);
      }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // the reads of V are done before the next copies overwrite it
    asm volatile("" ::: "memory");
  }

  // ---- merge the waves: O = sum_w 2^(m_w - m) O_w / sum_w 2^(m_w - m) l_w
  if (hf == 0) {
    m_sh[wave][col] = m_run;
    l_sh[wave][col] = l_run;
  }
  __syncthreads();
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) mx = fmaxf(mx, m_sh[w][col]);
  const float wscale = (m_run == -INFINITY) ? 0.f : exp2f(m_run - mx);
  float lt = 0.f;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) lt += (m_sh[w][col] == -INFINITY) ? 0.f : l_sh[w][col] * exp2f(m_sh[w][col] - mx);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // log-sum-exp of the row's scaled scores in natural units, for a backward that reuses it
  if (LSE && mode == MODE_FULL && wave == 0 && hf == 0 && r0 + col < Tq)
    LSE[((int64_t)b * Tq + r0 + col) * Hq + h] = (mx + log2f(lt)) * 0.6931471805599453f;
  // scaled partial outputs through LDS (fp32 [wave][row][dims], rows skewed; in the V^T area):
  // accumulators i..i+3 of a dim tile are 4 consecutive dims, written as one 16-byte store
  // (every wave has left its tile loop at the barrier above, so the table and V areas are free)
  float* part = lds;                                          // NWAVE x RT x PART_STRIDE floats
  const float sc = mode == MODE_FULL ? wscale * inv : wscale;   // partial modes stay unnormalised
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int dim = 32 * dt + 8 * i4 + 4 * hf;
      *reinterpret_cast<float4*>(&part[(wave * RT + col) * PART_STRIDE + dim]) =
          make_float4(oacc[dt][4 * i4] * sc, oacc[dt][4 * i4 + 1] * sc, oacc[dt][4 * i4 + 2] * sc,
                      oacc[dt][4 * i4 + 3] * sc);
    }
  __syncthreads();
  // thread -> (row, 8 dims): sum the waves' parts and write 8 contiguous floats
  for (int x = tid; x < RT * (D / 8); x += THREADS) {
    const int row_ = x / (D / 8), d0 = (x % (D / 8)) * 8;
    if (r0 + row_ >= Tq) continue;
    const int64_t ri = ((int64_t)b * Tq + r0 + row_) * Hq + h;     // (query, row, q-head)
    float* out = O + ri * D + d0;
    // partial modes: the row's merged max (log2 units of the pre-scaled scores) and sum
    float mxr = -INFINITY, ltr = 0.f;
    if (mode != MODE_FULL) {
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) mxr = fmaxf(mxr, m_sh[w][row_]);
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) ltr += (m_sh[w][row_] == -INFINITY) ? 0.f : l_sh[w][row_] * exp2f(m_sh[w][row_] - mxr);
    }
    // MEMORY: weights of this launch's sum and of the LOCAL partial (whose max is finite: every
    // row sees at least one local key)
    float a = 1.f, c = 0.f, rden = 1.f;
    if (mode == MODE_MEMORY) {
      const float ml = PML[2 * ri], ll = PML[2 * ri + 1];
      const float mt = fmaxf(mxr, ml);
      a = mxr == -INFINITY ? 0.f : exp2f(mxr - mt);
      c = exp2f(ml - mt);
      const float den = a * ltr + c * ll;
      rden = 1.f / den;
      if (LSE && d0 == 0) LSE[ri] = (mt + log2f(den)) * 0.6931471805599453f;
    }
    if (mode == MODE_LOCAL && d0 == 0) { PML[2 * ri] = mxr; PML[2 * ri + 1] = ltr; }
#pragma unroll
    for (int q4 = 0; q4 < 2; ++q4) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) {
        const float4 v = *reinterpret_cast<const float4*>(&part[(w * RT + row_) * PART_STRIDE + d0 + 4 * q4]);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      if (mode == MODE_LOCAL) {
        *reinterpret_cast<float4*>(PO + ri * D + d0 + 4 * q4) = acc;
      } else {
        if (mode == MODE_MEMORY) {
          const float4 pl = *reinterpret_cast<const float4*>(PO + ri * D + d0 + 4 * q4);
          acc.x = (a * acc.x + c * pl.x) * rden; acc.y = (a * acc.y + c * pl.y) * rden;
          acc.z = (a * acc.z + c * pl.z) * rden; acc.w = (a * acc.w + c * pl.w) * rden;
        }
        *reinterpret_cast<float4*>(out + 4 * q4) = acc;
      }
    }
  }
}

}  // namespace

namespace {
// ---------------------------------------------------------------- few query rows
// For decoding (Tq <= DEC_MAX_ROWS) one matrix-core tile would use 1 of its 32 rows.  Here a
// workgroup owns one (query row, q-head) and one lane owns one key: lanes form the key's
// score in fp32 (memory keys as given, local keys rotated from the LDS cos/sin table), the
// workgroup takes the softmax, and the output is summed over V rows that every thread loads into
// registers at the start (16 bytes of each of its keys), so their latency hides behind the scores.
// Used when every key fits: Mmax + Tl <= DEC_MAX_KEYS and Tl <= TAB_POS.
constexpr int DEC_THREADS = 512;             // two waves per SIMD
constexpr int DEC_LPK = 8;                    // lanes per key in the score pass (16 dims each)
constexpr int DEC_KPP = DEC_THREADS / DEC_LPK;   // keys per pass
constexpr int DEC_MAX_KEYS = DEC_THREADS;     // one key per lane in the softmax
constexpr int DEC_PASSES = DEC_MAX_KEYS / DEC_KPP;
constexpr int DEC_VSLOTS = DEC_THREADS / 16;  // V: 16 lanes per key row (16 bytes each), key slots
constexpr int DEC_VPT = DEC_MAX_KEYS / DEC_VSLOTS;   // keys per thread in the weighted sum
constexpr int DEC_MAX_ROWS = 4;
constexpr int DEC_WAVES = DEC_THREADS / 64;

__global__ void __launch_bounds__(DEC_THREADS, 1)
attn_decode_kernel(const uint16_t* __restrict__ Q, int Tq, int Hq, const uint16_t* __restrict__ Kloc,
                   const uint16_t* __restrict__ Vloc, int Tl, int Hkv, const uint16_t* __restrict__ Kmem,
                   const uint16_t* __restrict__ Vmem, int64_t mstride, int Mmax, const int32_t* __restrict__ mem_len,
                   int rope_offset, const RopeTables tabs, float scale_log2e, float* __restrict__ O,
                   float* __restrict__ LSE) {
  // one area: the cos/sin table (positions rope_offset + p, p < TAB_POS) while the scores are
  // formed, then the key slots' partial weighted sums [slot][dim]
  constexpr int TAB_BYTES = (int)sizeof(float2) * TAB_POS * (D / 2 + 2);
  constexpr int PV_BYTES = (int)sizeof(float) * DEC_VSLOTS * D;
  __shared__ __attribute__((aligned(16))) uint8_t area[TAB_BYTES > PV_BYTES ? TAB_BYTES : PV_BYTES];
  float2 (*cs_tab)[D / 2 + 2] = reinterpret_cast<float2 (*)[D / 2 + 2]>(area);
  float (*pv)[D] = reinterpret_cast<float (*)[D]>(area);
  __shared__ float qs[D];
  __shared__ float ps[DEC_MAX_KEYS];
  __shared__ float red[2][DEC_WAVES];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (Hq / Hkv);
  const int n_loc = (Tl - Tq) + i + 1;            // local keys this row sees
  // Loads in the order their data is needed (vector loads complete in order): the memory length,
  // the query pair and the table's constants before the key and value rows, so that the set-up
  // below waits for those alone.
  int M = mem_len[b];
  const int qt = tid & (D / 2 - 1);
  const uint16_t* qrow = Q + (((int64_t)b * Tq + i) * Hq + h) * D;
  const uint16_t q_x1 = qrow[qt], q_x2 = qrow[qt + D / 2];
  const double q_rev = tabs.rev[qt];
  const int fi = tid & (D / 2 - 1), sg = tid / (D / 2);
  static_assert(DEC_THREADS / (D / 2) * TAB_SEG >= TAB_POS, "the segments cover the table");
  const bool tab_thread = sg < TAB_POS / TAB_SEG && sg * TAB_SEG < n_loc;
  // every thread loads (segment index wrapped), so no load sits behind a branch
  const float2 t_st = tabs.start[sg & (TAB_POS / TAB_SEG - 1)][fi], t_d1 = tabs.step[fi], t_d8 = tabs.step8[fi];
  if (M < 0) M = 0;
  if (M > Mmax) M = Mmax;
  const int n = M + n_loc;                        // <= Mmax + Tl <= DEC_MAX_KEYS (checked at launch)

  auto key_row = [&](int key, const uint16_t* mem, const uint16_t* loc) {
    return key < M ? mem + ((int64_t)b * Mmax + key) * mstride + (int64_t)g * D
                   : loc + (((int64_t)b * Tl + (key - M)) * Hkv + g) * D;
  };
  // key rows, loaded up front and coalesced: 8 lanes per key, lane `sub` holds dims [8 sub, 8 sub + 8)
  // and their rotation partners [64 + 8 sub, 64 + 8 sub + 8); pass r covers keys DEC_KPP r + tid / 8
  const int sub = tid & (DEC_LPK - 1), kslot = tid / DEC_LPK;
  uint4 kr[DEC_PASSES][2];
#pragma unroll
  for (int r = 0; r < DEC_PASSES; ++r) {
    // keys past n read key n - 1 (unconditional loads keep the waits' counts exact); unused
    const int key = kslot + DEC_KPP * r;
    const uint16_t* kp = key_row(key < n ? key : n - 1, Kmem, Kloc);
    kr[r][0] = *reinterpret_cast<const uint4*>(kp + 8 * sub);
    kr[r][1] = *reinterpret_cast<const uint4*>(kp + D / 2 + 8 * sub);
  }
  // V rows for the weighted sum, also up front: key slot vs = tid / 16 holds keys vs, vs + 32, ...,
  // lane vd = tid % 16 dims [8 vd, 8 vd + 8) of each (a wave reads four 256-byte rows at a time)
  const int vslot = tid >> 4, vd = tid & 15;
  uint4 vr[DEC_VPT];
#pragma unroll
  for (int u = 0; u < DEC_VPT; ++u) {
    const int key = vslot + DEC_VSLOTS * u;       // past n: key n - 1 again, with weight zero
    vr[u] = *reinterpret_cast<const uint4*>(key_row(key < n ? key : n - 1, Vmem, Vloc) + 8 * vd);
  }
  // the query row, rotated at its position and pre-scaled by scale * log2(e)
  if (tid < D / 2) {
    const float x1 = __uint_as_float((uint32_t)q_x1 << 16), x2 = __uint_as_float((uint32_t)q_x2 << 16);
    float c, sn;
    rope_cs(rope_offset + (Tl - Tq) + i, q_rev, &c, &sn);
    qs[tid] = (x1 * c - x2 * sn) * scale_log2e;
    qs[tid + D / 2] = (x2 * c + x1 * sn) * scale_log2e;
  }
  // cos/sin table of the local keys' positions (as the matrix-core kernel builds it)
  if (tab_thread) fill_cs_segment(cs_tab, fi, sg * TAB_SEG, n_loc, t_st, t_d1, t_d8);
  __syncthreads();

  // scores: each key's 8 lanes rotate their pairs (local keys, from the table), take their share of
  // the dot product and sum it over the 8 lanes; the first lane stores the score
#pragma unroll
  for (int r = 0; r < DEC_PASSES; ++r) {
    const int key = kslot + DEC_KPP * r;
    if (DEC_KPP * r < n) {                        // uniform: some key of this pass exists
      float part = 0.f;
      if (key < n) {
        const uint4 a4 = kr[r][0], c4 = kr[r][1];
        float lo[8] = {bf16_lo(a4.x), bf16_hi(a4.x), bf16_lo(a4.y), bf16_hi(a4.y),
                       bf16_lo(a4.z), bf16_hi(a4.z), bf16_lo(a4.w), bf16_hi(a4.w)};
        float hi[8] = {bf16_lo(c4.x), bf16_hi(c4.x), bf16_lo(c4.y), bf16_hi(c4.y),
                       bf16_lo(c4.z), bf16_hi(c4.z), bf16_lo(c4.w), bf16_hi(c4.w)};
        if (key >= M) {
          const float4* t = reinterpret_cast<const float4*>(&cs_tab[key - M][8 * sub]);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 v = t[q4];
            float x1 = lo[2 * q4], x2 = hi[2 * q4];
            lo[2 * q4] = x1 * v.x - x2 * v.y; hi[2 * q4] = x2 * v.x + x1 * v.y;
            x1 = lo[2 * q4 + 1]; x2 = hi[2 * q4 + 1];
            lo[2 * q4 + 1] = x1 * v.z - x2 * v.w; hi[2 * q4 + 1] = x2 * v.z + x1 * v.w;
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) part += lo[e] * qs[8 * sub + e] + hi[e] * qs[D / 2 + 8 * sub + e];
      }
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      part += __shfl_xor(part, 4);
      if (sub == 0 && key < n) ps[key] = part;
    }
  }
  __syncthreads();
  float sc[1] = {tid < n ? ps[tid] : -INFINITY};
  // softmax over the row's keys: block max, then the block sum of exp2(score - max)
  float m = sc[0];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[0][wave] = m;
  __syncthreads();                                // also: every table read is done
  float mx = red[0][0];
#pragma unroll
  for (int w = 1; w < DEC_WAVES; ++w) mx = fmaxf(mx, red[0][w]);
  const float p = tid < n ? exp2f(sc[0] - mx) : 0.f;
  ps[tid] = p;                                    // each lane rewrites only its own score
  float l = p;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
  if (lane == 0) red[1][wave] = l;
  __syncthreads();
  float lt = 0.f;
#pragma unroll
  for (int w = 0; w < DEC_WAVES; ++w) lt += red[1][w];
  // O = sum_j p_j v_j / l: each thread sums its key slot's keys over its 8 dims (keys past n hold
  // zero rows and zero weights), then the slots' sums are added in order through LDS
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < DEC_VPT; ++u) {
    const int key = vslot + DEC_VSLOTS * u;
    if (DEC_VSLOTS * u < n) {                     // uniform: some key of this round exists
      const float w = key < n ? ps[key] : 0.f;
      const uint4 v = vr[u];
      acc[0] += w * bf16_lo(v.x); acc[1] += w * bf16_hi(v.x);
      acc[2] += w * bf16_lo(v.y); acc[3] += w * bf16_hi(v.y);
      acc[4] += w * bf16_lo(v.z); acc[5] += w * bf16_hi(v.z);
      acc[6] += w * bf16_lo(v.w); acc[7] += w * bf16_hi(v.w);
    }
  }
  *reinterpret_cast<float4*>(&pv[vslot][8 * vd]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(&pv[vslot][8 * vd + 4]) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();
  if (tid < D) {
    float sum = 0.f;
#pragma unroll 8
    for (int sl = 0; sl < DEC_VSLOTS; ++sl) sum += pv[sl][tid];
    const float inv = 1.f / lt;
    const int64_t ri = ((int64_t)b * Tq + i) * Hq + h;
    O[ri * D + tid] = sum * inv;
    if (LSE && tid == 0) LSE[ri] = (mx + log2f(lt)) * 0.6931471805599453f;
  }
}
}  // namespace

namespace {
int launch_attn_mode(const uint16_t* Q, int B, int Tq, int Hq, const uint16_t* Kloc, const uint16_t* Vloc,
                     int Tl, int Hkv, const uint16_t* Kmem, const uint16_t* Vmem, int64_t mem_entry_stride,
                     int Mmax, const int32_t* mem_len, int rope_offset, double rope_base, float scale,
                     float* O, float* lse, int mode, float* PO, float* PML, hipStream_t stream) {
  dim3 grid((unsigned)((Tq + RT - 1) / RT), (unsigned)Hq, (unsigned)B);
  const float scale_log2e = scale * 1.4426950408889634f;
  // RoPE constants in fp64: angle of position p at frequency i in revolutions, reduced to
  // [-1/2, 1/2] before cos/sin (the same reduction the device fallback uses).  They depend on
  // (rope_offset, rope_base) only; the last set is kept per host thread, since recomputing them
  // (~700 fp64 transcendentals) costs about as much host time as a decode call's GPU time.
  struct CachedTables { bool valid; int offset; double base; RopeTables t; };
  static thread_local CachedTables cache{false, 0, 0.0, {}};
  if (!cache.valid || cache.offset != rope_offset || cache.base != rope_base) {
    RopeTables& tb = cache.t;
    const double two_pi = 6.283185307179586;
    for (int i = 0; i < D / 2; ++i) {
      tb.rev[i] = pow(rope_base, -2.0 * i / D) / two_pi;
      auto cs = [&](double pos) {
        double r = pos * tb.rev[i];
        r -= rint(r);
        return make_float2((float)cos(two_pi * r), (float)sin(two_pi * r));
      };
      for (int sg = 0; sg < TAB_POS / TAB_SEG; ++sg) tb.start[sg][i] = cs((double)rope_offset + TAB_SEG * sg);
      tb.step[i] = cs(1.0);
      tb.step8[i] = cs(8.0);
    }
    cache.valid = true;
    cache.offset = rope_offset;
    cache.base = rope_base;
  }
  const RopeTables& tabs = cache.t;
  if (mode == MODE_FULL && Tq <= DEC_MAX_ROWS && Tl <= TAB_POS && (int64_t)Mmax + Tl <= DEC_MAX_KEYS) {
    hipLaunchKernelGGL(attn_decode_kernel, dim3((unsigned)Tq, (unsigned)Hq, (unsigned)B), dim3(DEC_THREADS), 0,
                       stream, Q, Tq, Hq, Kloc, Vloc, Tl, Hkv, Kmem, Vmem, mem_entry_stride, Mmax, mem_len,
                       rope_offset, tabs, scale_log2e, O, lse);
    MSA_CHECK_LAUNCH();
    return MSA_OK;
  }
  hipLaunchKernelGGL(attn_mfma_kernel, grid, dim3(THREADS), 0, stream, Q, Tq, Hq, Kloc, Vloc, Tl, Hkv, Kmem,
                     Vmem, mem_entry_stride, Mmax, mem_len, rope_offset, tabs, scale_log2e, O, lse, mode, PO, PML);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}
}  // namespace

int launch_attn(const uint16_t* Q, int B, int Tq, int Hq, const uint16_t* Kloc, const uint16_t* Vloc,
                int Tl, int Hkv, const uint16_t* Kmem, const uint16_t* Vmem, int64_t mem_entry_stride,
                int Mmax, const int32_t* mem_len, int rope_offset, double rope_base, float scale,
                float* O, float* lse, hipStream_t stream) {
  return launch_attn_mode(Q, B, Tq, Hq, Kloc, Vloc, Tl, Hkv, Kmem, Vmem, mem_entry_stride, Mmax, mem_len, rope_offset,
                          rope_base, scale, O, lse, MODE_FULL, nullptr, nullptr, stream);
}

int launch_attn_local(const uint16_t* Q, int B, int Tq, int Hq, const uint16_t* Kloc, const uint16_t* Vloc, int Tl,
                      int Hkv, int rope_offset, double rope_base, float scale, float* part_O, float* part_ml,
                      hipStream_t stream) {
  return launch_attn_mode(Q, B, Tq, Hq, Kloc, Vloc, Tl, Hkv, nullptr, nullptr, 0, 0, nullptr, rope_offset,
                          rope_base, scale, nullptr, nullptr, MODE_LOCAL, part_O, part_ml, stream);
}

int launch_attn_memory(const uint16_t* Q, int B, int Tq, int Hq, int Tl, int Hkv, const uint16_t* Kmem,
                       const uint16_t* Vmem, int64_t mem_entry_stride, int Mmax, const int32_t* mem_len,
                       int rope_offset, double rope_base, float scale, const float* part_O, const float* part_ml,
                       float* O, float* lse, hipStream_t stream) {
  return launch_attn_mode(Q, B, Tq, Hq, nullptr, nullptr, Tl, Hkv, Kmem, Vmem, mem_entry_stride, Mmax, mem_len,
                          rope_offset, rope_base, scale, O, lse, MODE_MEMORY, const_cast<float*>(part_O),
                          const_cast<float*>(part_ml), stream);
}

}  // namespace msa
