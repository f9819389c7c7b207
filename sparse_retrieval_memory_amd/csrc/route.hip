// Routing scan: chunk relevance of every pooled router key, then document max.
//
// What is computed (b-lab.team summary of MSA, sec. 1, Scalable Sparse
// Attention; medium write-up, sec. 2): for every pooled chunk g,
//   chunk[b,g] = max_t (1/H) sum_h cos(Qr[b,t,h], Krbar[g,h])
// and a document's score is the max over its chunks.  The scan reads the whole
// HBM-resident Krbar store once per call (the only O(L) online step), so the
// kernels are built around streaming it at HBM rate:
//
//  * Every row count takes the matrix cores: each workgroup keeps 128 router rows
//    resident in registers (8 waves: 4 row tiles of 32 x 2 head groups, bf16
//    MFMA A operands) and streams tiles of 32 chunks (64 KB for 8 heads)
//    through LDS with asynchronous global->LDS DMA, double buffered; chunk
//    rows are skewed by 16 bytes (XOR-swizzled pieces for H <= 2) so the
//    MFMA B-operand reads are bank-conflict free.  Per head: 8 x
//    v_mfma_f32_32x32x16_bf16 on the raw bf16 operands (exact products, fp32
//    accumulation), then an fp32 epilogue multiplies by 1/|q| and 1/|k| and
//    adds into the head sum (overlapped with the next head's MFMAs); the
//    token max is a register max plus one cross-lane step, combined across
//    waves/workgroups with an integer atomicMax on an order-preserving
//    encoding (deterministic).
//    For 8 heads (when every wave has rows) the tile is split into its two
//    halves of heads, which stream through a ring of four half-tile LDS buffers
//    with three halves in flight (route_ring8_kernel below): 3-5% faster than
//    the double-buffered whole tile at 100M tokens and at batch 16.
//    With few rows the idle row tiles only issue copies, and the scan streams at
//    the memory's rate (a VALU kernel with one thread per (chunk, head) was 1.1x
//    to 3.4x slower for 1 to 15 rows and has been removed).
//
// Normalisation is applied in fp32 after the exact bf16 dot products instead
// of rounding normalised vectors to bf16, which would move scores by ~1e-3.
#include "msa_internal.h"

#include <hip/hip_runtime.h>
#include <math.h>

namespace msa {
namespace {

constexpr int D = 128;
constexpr int TC = 32;   // chunks per MFMA tile (MFMA N)
constexpr int NW = 4;    // waves per MFMA workgroup
constexpr int RW = 32;   // router rows per wave (MFMA M)

// p[0, n) = v; p is 16-byte aligned (the route workspace), so whole 16-byte stores
// cover all but the last n % 4 words.
__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n4 = n >> 2;
  const uint4 q = make_uint4(v, v, v, v);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    reinterpret_cast<uint4*>(p)[i] = q;
  const int64_t t = (n4 << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) p[t] = v;
}

__device__ __forceinline__ float sq_norm_piece(uint4 v, float acc) {
  acc = dot2_bf16(v.x, v.x, acc);
  acc = dot2_bf16(v.y, v.y, acc);
  acc = dot2_bf16(v.z, v.z, acc);
  acc = dot2_bf16(v.w, v.w, acc);
  return acc;
}

__device__ __forceinline__ float inv_norm(float ss) { return ss > 0.f ? 1.0f / sqrtf(ss) : 0.f; }
// hardware reciprocal square root (about 1 ulp): used on the scan's hot path
__device__ __forceinline__ float inv_norm_fast(float ss) { return ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f; }

// ------------------------------------------------------------------ MFMA path
// Workgroup = 4 row tiles x HS head groups = 8 waves (H >= 2), two per SIMD:
// wave (rt, hs) keeps rows [32 rt, 32 rt + 32) of its row block and heads
// [hs*HPW, (hs+1)*HPW) resident as MFMA A operands (128 VGPRs for H = 8), so
// one wave's MFMAs overlap the other's epilogue.  The two head groups of a
// row tile add their partial head sums through LDS before the token max; the
// two waves take turns finishing a tile, which lets a single exchange buffer
// ride on the next tile's barrier instead of needing one of its own.
template <int H>
struct Cfg {
  static constexpr int ROW_BYTES = H * D * 2;       // one pooled chunk, all heads
  static constexpr int PIECES = ROW_BYTES / 16;     // 16-byte pieces per chunk row
  static constexpr int BYTES = TC * ROW_BYTES;      // tile bytes in HBM: 8 KB * H
  // LDS row stride: for H >= 4 each chunk row is skewed by 16 bytes so the 32
  // lanes of an MFMA B-operand read (one chunk each, same offset) hit distinct
  // banks; for H <= 2 (a DMA instruction spans several rows) rows are packed
  // and the 16-byte pieces are XOR-swizzled instead
  static constexpr bool SKEW = PIECES >= 64;
  static constexpr int ROW_STRIDE = SKEW ? ROW_BYTES + 16 : ROW_BYTES;
  static constexpr int TILE_LDS = TC * ROW_STRIDE;
  static constexpr int RK_BYTES = TC * H * 4;       // the tile's 1/|k| block (fp32 [TC][H])
  static constexpr int HS = H >= 2 ? 2 : 1;         // head groups per row tile
  static constexpr int HPW = H / HS;                // heads per wave
  static constexpr int NWAVES = NW * HS;
  static constexpr int THREADS = 64 * NWAVES;
  static constexpr int DMA_ITERS = BYTES / (16 * THREADS);
};

// Source of one chunk tile's copies: the tile's first row (wave-uniform, kept in
// scalar registers) and the last valid row index within the tile.  Chunks past
// the end are clamped to the last chunk (their results are never written).
struct TileSrc {
  const uint8_t* base;
  int nmax;
};
template <int H>
__device__ __forceinline__ TileSrc tile_src(const uint8_t* __restrict__ kr, int64_t n_chunks, int64_t tile) {
  const int64_t left = n_chunks - 1 - tile * TC;
  const uint64_t base = (uint64_t)(kr + tile * TC * Cfg<H>::ROW_BYTES);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  return TileSrc{(const uint8_t*)(((uint64_t)hi << 32) | lo),
                 __builtin_amdgcn_readfirstlane(left < TC - 1 ? (int)left : TC - 1)};
}

// Asynchronous copy of piece `i` (of Cfg::DMA_ITERS) of a chunk tile into `lds`:
// each wave instruction moves 1 KB of contiguous global memory (half a chunk
// row for H = 8) into the row's skewed LDS slot; for H <= 2 LDS slot j instead
// holds piece (j % PIECES) ^ (n & 15) of chunk n = j / PIECES.
template <int H, int POL>
__device__ __forceinline__ void issue_piece(const TileSrc& src, uint8_t* lds, int wave, int lane, int i) {
  using CF = Cfg<H>;
  const int slot0 = (i * CF::NWAVES + wave) * 64;     // wave-uniform
  if constexpr (CF::SKEW) {
    const int n = slot0 / CF::PIECES;                 // one chunk per wave instruction: uniform
    const int ne = n < src.nmax ? n : src.nmax;
    const uint8_t* sb = src.base + ne * CF::ROW_BYTES + (slot0 % CF::PIECES) * 16;
    dma16<POL>(sb + (uint32_t)lane * 16u, lds + n * CF::ROW_STRIDE + (slot0 % CF::PIECES) * 16);
  } else {
    const int n = (slot0 + lane) / CF::PIECES;
    const int pp = (slot0 + lane) % CF::PIECES;
    const int ne = n < src.nmax ? n : src.nmax;
    const uint32_t off = (uint32_t)((pp ^ (n & 15)) * 16);
    dma16<POL>(src.base + ne * CF::ROW_BYTES + off, lds + slot0 * 16);
  }
}

// With stored norms (H >= 4) the tile's fp32 [TC][H] block of 1/|k| goes into
// `lds_rk` (one instruction of the last wave; 16-byte granules never straddle a
// chunk boundary for H >= 4, so clamping is per chunk).
template <int H, int POL>
__device__ __forceinline__ void issue_norms(const float* __restrict__ knorm, int64_t n_chunks, int64_t tile,
                                            float* lds_rk, int wave, int lane) {
  using CF = Cfg<H>;
  static_assert(H >= 4, "stored norms need 16-byte granules within one chunk");
  constexpr int GR = CF::RK_BYTES / 16;               // granules per tile (<= 64)
  const bool full = (tile + 1) * TC <= n_chunks;
  if (wave == CF::NWAVES - 1 && lane < GR) {
    if (full) {
      const uint64_t base = (uint64_t)(knorm + tile * TC * H);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
      dma16<POL>((const uint8_t*)(((uint64_t)hi << 32) | lo) + (uint32_t)lane * 16u, lds_rk);
    } else {
      const int n = lane * 4 / H;
      const int64_t g = (tile * TC + n < n_chunks) ? tile * TC + n : n_chunks - 1;
      dma16<POL>(knorm + g * H + (lane * 4) % H, lds_rk);
    }
  }
}

// The whole tile (and its norms block) at once.
template <int H, bool NORMS, int POL>
__device__ __forceinline__ void issue_tile(const uint8_t* __restrict__ kr, const float* __restrict__ knorm,
                                           int64_t n_chunks, int64_t tile, uint8_t* lds, float* lds_rk,
                                           int wave, int lane) {
  const TileSrc src = tile_src<H>(kr, n_chunks, tile);
#pragma unroll
  for (int i = 0; i < Cfg<H>::DMA_ITERS; ++i) issue_piece<H, POL>(src, lds, wave, lane, i);
  if constexpr (NORMS) issue_norms<H, POL>(knorm, n_chunks, tile, lds_rk, wave, lane);
}

// Token max of a finished 32-row x 32-chunk head sum, then the chunk's atomic max.
__device__ __forceinline__ void finish_tile(const f32x16_t& sacc, int half, int nb, int t0, int T, int b,
                                            int64_t tile, int64_t n_chunks, float inv_h, uint32_t* chunk_enc) {
  // accumulator i of this lane holds row 8*(i/4) + 4*half + i%4
  float v = -INFINITY;
  if (t0 + RW <= T) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v = fmaxf(v, sacc[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * (i >> 2) + 4 * half + (i & 3);
      if (t0 + row < T) v = fmaxf(v, sacc[i]);
    }
  }
  v = fmaxf(v, __shfl_xor(v, 32));
  const int64_t g = tile * TC + nb;
  if (half == 0 && g < n_chunks) atomicMax(&chunk_enc[(int64_t)b * n_chunks + g], enc_f32(v * inv_h));
}

// One tile of the MFMA scan: wait for `cur` (filled by the previous step),
// start filling `nxt` with the following tile, finish the previous tile's head
// sum if this wave is its receiver, then score `cur`.  `cur`/`nxt` are
// distinct LDS arrays so the compiler can see that reading one does not
// depend on the DMA into the other.  PAR is the tile's parity within the
// workgroup's range: on even tiles head group 1 sends and group 0 finishes,
// on odd tiles the other way round.
template <int H, bool NORMS, int PAR, int POL>
__device__ __forceinline__ void mfma_tile_step(const uint8_t* __restrict__ kr, const float* __restrict__ knorm,
                                               int64_t n_chunks, int64_t tile, bool has_prev, bool has_next,
                                               const uint8_t* cur, const float* cur_rk, uint8_t* nxt, float* nxt_rk,
                                               float (*lds_rq)[RW], f32x4_t* xchg,
                                               const bf16x8_t (&qf)[Cfg<H>::HPW][8], f32x16_t& sprev,
                                               bool wave_active, int hs, int b, int t0, int T,
                                               uint32_t* chunk_enc, int wave, int lane) {
  using CF = Cfg<H>;
  const int half = lane >> 5;
  const int nb = lane & 31;                   // this lane's chunk column in the tile
  wait_vmem_all();
  lds_barrier();                              // tile visible; previous tile fully consumed
  // The next tile's copies are interleaved with this tile's first MFMAs (one after
  // each), so the waves do not stall on issuing them while the matrix unit idles.
  // On the last step the copy re-reads the current tile into the unused buffer
  // instead of branching around every instruction.
  const TileSrc src = tile_src<H>(kr, n_chunks, has_next ? tile + 1 : tile);
  if constexpr (NORMS) {
    if (has_next) issue_norms<H, POL>(knorm, n_chunks, tile + 1, nxt_rk, wave, lane);
  }
  if (!wave_active) {
#pragma unroll
    for (int i = 0; i < CF::DMA_ITERS; ++i) issue_piece<H, POL>(src, nxt, wave, lane, i);
  }

  f32x4_t* x = xchg + lane;                   // layout [q4][lane]: 16-byte lane stride, conflict-free
  if (CF::HS == 2 && has_prev && wave_active && hs == (PAR == 0 ? 1 : 0)) {
    // receiver of the previous tile (parity 1 - PAR): add the sender's half and finish it
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4_t o = x[q4 * 64];
      sprev[4 * q4] += o[0]; sprev[4 * q4 + 1] += o[1]; sprev[4 * q4 + 2] += o[2]; sprev[4 * q4 + 3] += o[3];
    }
    finish_tile(sprev, half, nb, t0, T, b, tile - 1, n_chunks, 1.0f / H, chunk_enc);
  }
  if (!wave_active) return;

  f32x16_t sacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
  const uint8_t* brow = cur + nb * CF::ROW_STRIDE;
  // One head: 8 B-operand reads and the MFMA chain over the 128 dims (and, without
  // stored norms, |k|^2 of this lane's half of chunk nb from the same reads).
  auto head_mfma = [&](int hh, f32x16_t& acc, float& ss) {
    const int h = hs * CF::HPW + hh;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    ss = 0.f;
#pragma unroll
    for (int k4 = 0; k4 < 8; k4 += 4) {
      bf16x8_t bv[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int lp = 16 * h + 2 * (k4 + ks) + half;
        const int pp = CF::SKEW ? lp : (lp ^ (nb & 15));
        bv[ks] = *reinterpret_cast<const bf16x8_t*>(brow + pp * 16);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[hh][k4 + ks], bv[ks], acc, 0, 0, 0);
        if constexpr (!NORMS) ss = sq_norm_piece(__builtin_bit_cast(uint4, bv[ks]), ss);
        const int mf = hh * 8 + k4 + ks;      // MFMA number within the step (compile time)
        if (mf < CF::DMA_ITERS) issue_piece<H, POL>(src, nxt, wave, lane, mf);
      }
    }
  };
  // Epilogue of one head: scale by 1/|k| (column) and 1/|q| (row) and add into the head sum.
  // 1/|q| of the lane's 16 rows for head hh: loaded at the start of the pipeline step,
  // ahead of the next head's MFMA chain, so the epilogue does not wait on LDS.
  auto load_rq = [&](int hh, float4 (&rq)[4]) {
    const int h = hs * CF::HPW + hh;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) rq[q4] = *reinterpret_cast<const float4*>(&lds_rq[h][8 * q4 + 4 * half]);
  };
  auto head_epilogue = [&](int hh, const f32x16_t& acc, float ss, const float4 (&rqv)[4]) {
    const int h = hs * CF::HPW + hh;
    float rk;
    if constexpr (NORMS) {
      rk = cur_rk[nb * H + h];
    } else {
      ss += __shfl_xor(ss, 32);               // lanes l and l^32 hold the two halves of chunk nb
      rk = inv_norm_fast(ss);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 rq = rqv[q4];
      sacc[4 * q4 + 0] = fmaf(acc[4 * q4 + 0], rk * rq.x, sacc[4 * q4 + 0]);
      sacc[4 * q4 + 1] = fmaf(acc[4 * q4 + 1], rk * rq.y, sacc[4 * q4 + 1]);
      sacc[4 * q4 + 2] = fmaf(acc[4 * q4 + 2], rk * rq.z, sacc[4 * q4 + 2]);
      sacc[4 * q4 + 3] = fmaf(acc[4 * q4 + 3], rk * rq.w, sacc[4 * q4 + 3]);
    }
  };
  // Software pipeline over the heads: head hh + 1's MFMA chain is issued before head hh's
  // epilogue, so the matrix unit keeps working while the vector unit finishes the previous
  // head; at most two heads are in flight (a scheduling fence ends each step).
  f32x16_t acc_a, acc_b;
  float ss_a = 0.f, ss_b = 0.f;
  head_mfma(0, acc_a, ss_a);
#pragma unroll
  for (int hh = 0; hh < CF::HPW; ++hh) {
    f32x16_t& cur_acc = (hh & 1) ? acc_b : acc_a;
    f32x16_t& nxt_acc = (hh & 1) ? acc_a : acc_b;
    float& cur_ss = (hh & 1) ? ss_b : ss_a;
    float& nxt_ss = (hh & 1) ? ss_a : ss_b;
    float4 rqv[4];
    load_rq(hh, rqv);
    if (hh + 1 < CF::HPW) head_mfma(hh + 1, nxt_acc, nxt_ss);
    head_epilogue(hh, cur_acc, cur_ss, rqv);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (CF::HS == 2) {
    if (hs == (PAR == 0 ? 1 : 0)) {           // sender of this tile
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        x[q4 * 64] = f32x4_t{sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]};
    } else {
      sprev = sacc;                           // finished at the start of the next step
    }
  } else {
    finish_tile(sacc, half, nb, t0, T, b, tile, n_chunks, 1.0f / H, chunk_enc);
  }
}

template <int H, bool NORMS, int POL>
__global__ void __launch_bounds__(Cfg<H>::THREADS, 1)
route_mfma_kernel(const uint16_t* __restrict__ Qr, int B, int T, int RTq, int P, int S,
                  const uint16_t* __restrict__ Krbar, const float* __restrict__ knorm, int64_t n_chunks,
                  int64_t tiles_per_slice, uint32_t* __restrict__ chunk_enc) {
  using CF = Cfg<H>;
  // each buffer = the chunk tile followed by its 1/|k| block: one LDS object per
  // buffer, so the compiler's DMA tracking never has to order DMAs into
  // different objects (it would wait for the whole prefetch otherwise)
  constexpr int RKB = NORMS ? CF::RK_BYTES : 0;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[CF::TILE_LDS + RKB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[CF::TILE_LDS + RKB];
  float* rk_a = reinterpret_cast<float*>(lds_a + CF::TILE_LDS);
  float* rk_b = reinterpret_cast<float*>(lds_b + CF::TILE_LDS);
  __shared__ __attribute__((aligned(16))) float lds_rq[NW][H][RW];
  __shared__ __attribute__((aligned(16))) f32x4_t lds_x[NW][64 * 4];

  // XCD-aware block mapping: workgroups are dealt round-robin to the 8 XCDs;
  // keep the P row blocks of one chunk slice on the same XCD so they share
  // that XCD's L2 copy of the slice.
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int j = bid >> 3;
  const int p = j % P;
  const int s = (j / P) * 8 + xcd;
  if (s >= S) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, m = lane & 31;
  const int rtl = wave % NW;                  // row tile within the block
  const int hs = wave / NW;                   // head group
  const int rt = p * NW + rtl;                // global row tile
  const bool wave_active = rt < B * RTq;
  const int b = wave_active ? rt / RTq : 0;
  const int t0 = (rt % RTq) * RW;

  // --- resident router rows: A operands for this wave's heads and all k-steps
  bf16x8_t qf[CF::HPW][8];
  {
    const int t = t0 + m;
    const bool valid = wave_active && t < T;
    const uint16_t* qrow = Qr + ((int64_t)b * T + t) * H * D;
#pragma unroll
    for (int hh = 0; hh < CF::HPW; ++hh) {
      const int h = hs * CF::HPW + hh;
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (valid) v = *reinterpret_cast<const uint4*>(qrow + h * D + 16 * ks + 8 * half);
        qf[hh][ks] = __builtin_bit_cast(bf16x8_t, v);
        ss = sq_norm_piece(v, ss);
      }
      ss += __shfl_xor(ss, 32);
      if (half == 0) lds_rq[rtl][h][m] = inv_norm(ss);
    }
  }

  const int64_t n_tiles = (n_chunks + TC - 1) / TC;
  const int64_t tile_begin = (int64_t)s * tiles_per_slice;
  int64_t tile_end = tile_begin + tiles_per_slice;
  if (tile_end > n_tiles) tile_end = n_tiles;
  if (tile_begin >= tile_end) return;

  const uint8_t* kr = reinterpret_cast<const uint8_t*>(Krbar);
  f32x16_t sprev;
#pragma unroll
  for (int i = 0; i < 16; ++i) sprev[i] = 0.f;
  issue_tile<H, NORMS, POL>(kr, knorm, n_chunks, tile_begin, lds_a, rk_a, wave, lane);
  int64_t tile = tile_begin;
  for (; tile < tile_end; tile += 2) {
    mfma_tile_step<H, NORMS, 0, POL>(kr, knorm, n_chunks, tile, tile > tile_begin, tile + 1 < tile_end, lds_a, rk_a,
                                lds_b, rk_b, lds_rq[rtl], lds_x[rtl], qf, sprev, wave_active, hs, b, t0, T,
                                chunk_enc, wave, lane);
    if (tile + 1 < tile_end)
      mfma_tile_step<H, NORMS, 1, POL>(kr, knorm, n_chunks, tile + 1, true, tile + 2 < tile_end, lds_b, rk_b, lds_a,
                                  rk_a, lds_rq[rtl], lds_x[rtl], qf, sprev, wave_active, hs, b, t0, T,
                                  chunk_enc, wave, lane);
  }
  if constexpr (CF::HS == 2) {
    // finish the last tile: its parity decides which head group receives
    const int64_t last = tile_end - 1;
    const int par = (int)((last - tile_begin) & 1);
    lds_barrier();
    if (wave_active && hs == (par == 0 ? 0 : 1)) {
      f32x4_t* x = lds_x[rtl] + lane;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4_t o = x[q4 * 64];
        sprev[4 * q4] += o[0]; sprev[4 * q4 + 1] += o[1]; sprev[4 * q4 + 2] += o[2]; sprev[4 * q4 + 3] += o[3];
      }
      finish_tile(sprev, half, m, t0, T, b, last, n_chunks, 1.0f / H, chunk_enc);
    }
  }
  wait_vmem_all();                            // the last step's copy lands before the LDS is released
}

// ------------------------------------------------- 8 heads: a ring of half-tiles
// For H = 8 the tile of 32 chunks is cut into its two halves of rows (heads 0-3 and
// heads 4-7, 1 KB of every chunk row each) and the halves stream through a ring of
// four 32 KB LDS buffers.  A half is consumed by all eight waves in one sub-step:
// wave (row tile, hs) keeps heads {2hs, 2hs+1} of the first half and {4+2hs, 5+2hs}
// of the second resident, so every wave scores two heads per sub-step and the
// head sum of a tile is complete after its second half.  At sub-step j the copies
// of half-tile j + 3 go into the buffer freed by sub-step j - 1: three half-tiles
// (96 KB) are in flight while one is scored, against one 64 KB tile with two
// whole-tile buffers, so the scan no longer waits for the memory when a tile's
// scoring is shorter than the memory's latency.  Each wave waits only for its own
// copies of the half-tile it is about to score (the 8 younger copies, of the next
// two half-tiles, may stay in flight: vector loads complete in order), then the
// workgroup barrier makes everyone's copies visible.  The tile's 1/|k| block has a
// pair of its own buffers, filled one tile ahead.
constexpr int RING_ROW = 4 * D * 2;              // half a chunk row: 4 heads, 1 KB
constexpr int RING_STRIDE = RING_ROW + 16;       // skewed so B-operand reads hit distinct banks
constexpr int RING_LDS = TC * RING_STRIDE;       // one half-tile buffer
constexpr int RING_COPIES = TC / 8;              // copies per wave per half-tile (one chunk row half each)
constexpr int RING_VMCNT_YOUNGER = 2 * RING_COPIES;
static_assert(RING_VMCNT_YOUNGER == 8, "the wait below is written for 8 younger copies");

// The ring's copies are buffer loads into LDS written as inline assembly, so the compiler does not
// track them (its conservative tracking of LDS copies drained every copy in flight before reads of
// unrelated LDS data); the sub-steps wait for them explicitly.  Every operand is a register the copy
// does not outlive: the buffer resource, the scalar offset and M0 are scalars written right before
// it, and the lane offset (voff) is one register that holds lane * 16 for the whole kernel.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t ring_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r[0] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);   // stride 0
  r[2] = (int32_t)__builtin_amdgcn_readfirstlane(bytes);                           // range checked
  r[3] = 0x00020000;
  return r;
}
template <int POL, int BYTES>
__device__ __forceinline__ void ring_dma(const i32x4_t& rs, uint32_t soff, uint32_t voff, const void* lds) {
  // the LDS byte address (M0 takes the local address, not the generic one)
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds);
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  if constexpr (BYTES == 16 && POL == POL_NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :: "s"(m0v), "v"(voff), "s"(rs), "s"(so) : "memory", "m0");
  else if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(m0v), "v"(voff), "s"(rs), "s"(so) : "memory", "m0");
  else if constexpr (POL == POL_NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen nt lds"
                 :: "s"(m0v), "v"(voff), "s"(rs), "s"(so) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(m0v), "v"(voff), "s"(rs), "s"(so) : "memory", "m0");
}

// Copies of half-tile (tile, hf) into `lds`: wave w moves the hf half-rows of chunks w, w + 8, ...
// through a buffer resource on the tile's first row (rows past the store's end re-read its last
// row).  Tiles past the slice's end (te) get an empty resource: their copies, issued ahead so the
// waits keep their fixed count, touch no memory (the range check turns them into zeros).
struct RingSrc {
  i32x4_t rs;
  int last;                                    // last valid row of the tile
};
__device__ __forceinline__ RingSrc ring_src(const uint8_t* kr, int64_t n_chunks, int64_t tile, int64_t te) {
  const int64_t n_tiles = (n_chunks + TC - 1) / TC;
  const int64_t t = tile < n_tiles ? tile : n_tiles - 1;
  const int64_t left = n_chunks - 1 - t * TC;
  RingSrc r;
  r.rs = ring_rsrc(kr + t * TC * (2 * RING_ROW), tile < te ? TC * 2 * RING_ROW : 0u);
  r.last = __builtin_amdgcn_readfirstlane((int)(left < TC - 1 ? left : TC - 1));
  return r;
}
template <int POL>
__device__ __forceinline__ void ring_copy(const RingSrc& src, int hf, uint8_t* lds, int wave, uint32_t voff, int i) {
  int n = wave + 8 * i;
  n = n < src.last ? n : src.last;
  ring_dma<POL, 16>(src.rs, (uint32_t)(n * (2 * RING_ROW) + hf * RING_ROW), voff, lds + (wave + 8 * i) * RING_STRIDE);
}

// The tile's 1/|k| block, fp32 [32][8] = 1 KB: wave w copies quarter w % 4 (chunks 8q .. 8q + 7, 256 B)
// with a 4-byte-per-lane copy (waves 4-7 repeat waves 0-3, writing the same values).  voff4 =
// 4 lane + 256 q; lanes past the store's end read 0 (the buffer's range check), as does the whole
// block of a tile past the slice's end.
template <int POL>
__device__ __forceinline__ void ring_norms(const float* knorm, int64_t n_chunks, int64_t tile, int64_t te,
                                           float* lds_rk, int wave, uint32_t voff4) {
  const int64_t n_tiles = (n_chunks + TC - 1) / TC;
  const int64_t t = tile < n_tiles ? tile : n_tiles - 1;
  const int64_t rows = n_chunks - t * TC < TC ? n_chunks - t * TC : TC;   // the tile's rows in the store
  const i32x4_t rs = ring_rsrc(knorm + t * TC * 8, tile < te ? (uint32_t)(rows * 8 * 4) : 0u);
  ring_dma<POL, 4>(rs, 0u, voff4, lds_rk + 64 * (wave & 3));
}

// One sub-step: score half HF of tile `tile` from `cur` (ring slot J4 = j % 4, so HF = J4 & 1),
// start the copies of half-tile j + 3 into `nxt`, and (HF == 0) finish the previous tile if this
// wave is its receiver.  The wave of the first head group (hs = 0) receives and finishes every
// tile: the second group's waves, issued after it on the same SIMDs, reach the end of a
// sub-step ~10% later, so giving the finish to the first group balances the pair (1-2.5% faster
// than alternating the roles by tile parity, A/B on one box).
template <bool NORMS, int POL, int J4>
__device__ __forceinline__ void ring_sub_step(const uint8_t* __restrict__ kr, const float* __restrict__ knorm,
                                              int64_t n_chunks, int64_t tile, int64_t te, bool has_prev,
                                              const uint8_t* cur, uint8_t* nxt, const float* rk_cur,
                                              float* rk_next, float (*lds_rq)[RW], f32x4_t* xchg,
                                              const bf16x8_t (&qf)[4][8], f32x16_t& sacc, f32x16_t& sprev,
                                              int hs, int b, int t0, int T,
                                              uint32_t* chunk_enc, int wave, int lane,
                                              float4& rk4, uint32_t voff, uint32_t voff4) {
  constexpr int HF = J4 & 1;
  const int half = lane >> 5;
  const int nb = lane & 31;
  __builtin_amdgcn_s_waitcnt(0x0F78);         // vmcnt(8): this wave's copies of half-tile j are done
  asm volatile("" ::: "memory");
  lds_barrier();                              // everyone's copies visible; slot j - 1 fully consumed
  // half-tile j + 3: (tile + 1, 1 - HF) when HF == 0 ... (tile + 2, 0) when HF == 1
  const RingSrc csrc = ring_src(kr, n_chunks, HF == 0 ? tile + 1 : tile + 2, te);
  constexpr int CHF = 1 - HF;
  if constexpr (NORMS && HF == 0) {
    // this tile's 1/|k| for the wave's four heads, read before the next tile's block is requested
    const float2 lo = *reinterpret_cast<const float2*>(rk_cur + nb * 8 + 2 * hs);
    const float2 hi = *reinterpret_cast<const float2*>(rk_cur + nb * 8 + 4 + 2 * hs);
    rk4 = make_float4(lo.x, lo.y, hi.x, hi.y);
    ring_norms<POL>(knorm, n_chunks, tile + 1, te, rk_next, wave, voff4);
  }
  f32x4_t* x = xchg + lane;
  if constexpr (HF == 0) {
    if (has_prev && hs == 0) {
      // receiver of the previous tile: add the sender's half and finish it
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4_t o = x[q4 * 64];
        sprev[4 * q4] += o[0]; sprev[4 * q4 + 1] += o[1]; sprev[4 * q4 + 2] += o[2]; sprev[4 * q4 + 3] += o[3];
      }
      finish_tile(sprev, half, nb, t0, T, b, tile - 1, n_chunks, 1.0f / 8, chunk_enc);
    }
  }
  if constexpr (HF == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
  }
  const uint8_t* brow = cur + nb * RING_STRIDE;
  // head hl (0/1) of this sub-step: resident operand qf[2 HF + hl], global head h, local head in the half
  auto head_mfma = [&](int hl, f32x16_t& acc, float& ss) {
    const int hloc = 2 * hs + hl;             // head within the half-row
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    ss = 0.f;
#pragma unroll
    for (int k4 = 0; k4 < 8; k4 += 4) {
      bf16x8_t bv[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        bv[ks] = *reinterpret_cast<const bf16x8_t*>(brow + (16 * hloc + 2 * (k4 + ks) + half) * 16);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[2 * HF + hl][k4 + ks], bv[ks], acc, 0, 0, 0);
        if constexpr (!NORMS) ss = sq_norm_piece(__builtin_bit_cast(uint4, bv[ks]), ss);
        const int mf = hl * 8 + k4 + ks;
        if (mf < RING_COPIES) ring_copy<POL>(csrc, CHF, nxt, wave, voff, mf);
      }
    }
  };
  auto load_rq = [&](int hl, float4 (&rq)[4]) {
    const int h = 4 * HF + 2 * hs + hl;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) rq[q4] = *reinterpret_cast<const float4*>(&lds_rq[h][8 * q4 + 4 * half]);
  };
  auto head_epilogue = [&](int hl, const f32x16_t& acc, float ss, const float4 (&rqv)[4]) {
    const int h = 4 * HF + 2 * hs + hl;
    float rk;
    if constexpr (NORMS) {
      rk = HF == 0 ? (hl == 0 ? rk4.x : rk4.y) : (hl == 0 ? rk4.z : rk4.w);
    } else {
      ss += __shfl_xor(ss, 32);
      rk = inv_norm_fast(ss);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 rq = rqv[q4];
      sacc[4 * q4 + 0] = fmaf(acc[4 * q4 + 0], rk * rq.x, sacc[4 * q4 + 0]);
      sacc[4 * q4 + 1] = fmaf(acc[4 * q4 + 1], rk * rq.y, sacc[4 * q4 + 1]);
      sacc[4 * q4 + 2] = fmaf(acc[4 * q4 + 2], rk * rq.z, sacc[4 * q4 + 2]);
      sacc[4 * q4 + 3] = fmaf(acc[4 * q4 + 3], rk * rq.w, sacc[4 * q4 + 3]);
    }
  };
  f32x16_t acc_a, acc_b;
  float ss_a = 0.f, ss_b = 0.f;
  head_mfma(0, acc_a, ss_a);
  {
    float4 rqv[4];
    load_rq(0, rqv);
    head_mfma(1, acc_b, ss_b);
    head_epilogue(0, acc_a, ss_a, rqv);
  }
  {
    float4 rqv[4];
    load_rq(1, rqv);
    head_epilogue(1, acc_b, ss_b, rqv);
  }
  if constexpr (HF == 1) {
    if (hs == 1) {                            // sender of this tile
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        x[q4 * 64] = f32x4_t{sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]};
    } else {
      sprev = sacc;                           // finished at the start of the next tile
    }
  }
}

template <bool NORMS, int POL>
__global__ void __launch_bounds__(512, 1)
route_ring8_kernel(const uint16_t* __restrict__ Qr, int B, int T, int RTq, int P, int S,
                   const uint16_t* __restrict__ Krbar, const float* __restrict__ knorm, int64_t n_chunks,
                   int64_t tiles_per_slice, uint32_t* __restrict__ chunk_enc) {
  // four distinct LDS objects, so the compiler can tell which copies a read depends on
  __shared__ __attribute__((aligned(16))) uint8_t ring0[RING_LDS];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[RING_LDS];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[RING_LDS];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[RING_LDS];
  __shared__ __attribute__((aligned(16))) float rk0[NORMS ? TC * 8 : 4];
  __shared__ __attribute__((aligned(16))) float rk1[NORMS ? TC * 8 : 4];
  __shared__ __attribute__((aligned(16))) float lds_rq[NW][8][RW];
  __shared__ __attribute__((aligned(16))) f32x4_t lds_x[NW][64 * 4];

  const int bid = blockIdx.x;                 // XCD-aware mapping, as in route_mfma_kernel
  const int xcd = bid & 7;
  const int j0 = bid >> 3;
  const int p = j0 % P;
  const int s = (j0 / P) * 8 + xcd;
  if (s >= S) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, m = lane & 31;
  const int rtl = wave % NW;
  const int hs = wave / NW;
  const int rt = p * NW + rtl;                // < B * RTq: every wave has rows (B * RTq % 4 == 0)
  const int b = rt / RTq;
  const int t0 = (rt % RTq) * RW;

  // resident router rows: qf[0..1] = heads 2hs, 2hs+1; qf[2..3] = heads 4+2hs, 5+2hs
  bf16x8_t qf[4][8];
  {
    const int t = t0 + m;
    const bool valid = t < T;
    const uint16_t* qrow = Qr + ((int64_t)b * T + t) * 8 * D;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const int h = 4 * (hh >> 1) + 2 * hs + (hh & 1);
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (valid) v = *reinterpret_cast<const uint4*>(qrow + h * D + 16 * ks + 8 * half);
        qf[hh][ks] = __builtin_bit_cast(bf16x8_t, v);
        ss = sq_norm_piece(v, ss);
      }
      ss += __shfl_xor(ss, 32);
      if (half == 0) lds_rq[rtl][h][m] = inv_norm(ss);
    }
  }

  const int64_t n_tiles = (n_chunks + TC - 1) / TC;
  const int64_t tb = (int64_t)s * tiles_per_slice;
  int64_t te = tb + tiles_per_slice;
  if (te > n_tiles) te = n_tiles;
  if (tb >= te) return;

  const uint8_t* kr = reinterpret_cast<const uint8_t*>(Krbar);
  float4 rk4 = make_float4(0.f, 0.f, 0.f, 0.f);
  f32x16_t sacc, sprev;
#pragma unroll
  for (int i = 0; i < 16; ++i) { sacc[i] = 0.f; sprev[i] = 0.f; }
  // prologue: the tile's norms, then half-tiles 0, 1, 2 (the order the sub-steps' waits assume)
  const uint32_t voff = (uint32_t)lane * 16u;       // the lane's byte in a copied half-row
  const uint32_t voff4 = (uint32_t)lane * 4u + (uint32_t)(wave & 3) * 256u;   // ... in a norms block
  if constexpr (NORMS) ring_norms<POL>(knorm, n_chunks, tb, te, rk0, wave, voff4);
  {
    const RingSrc s0 = ring_src(kr, n_chunks, tb, te), s1 = ring_src(kr, n_chunks, tb + 1, te);
#pragma unroll
    for (int i = 0; i < RING_COPIES; ++i) ring_copy<POL>(s0, 0, ring0, wave, voff, i);
#pragma unroll
    for (int i = 0; i < RING_COPIES; ++i) ring_copy<POL>(s0, 1, ring1, wave, voff, i);
#pragma unroll
    for (int i = 0; i < RING_COPIES; ++i) ring_copy<POL>(s1, 0, ring2, wave, voff, i);
  }

#define MSA_RING_SUB(J4, TILE, CUR, NXT, RKC, RKN)                                                              \
  ring_sub_step<NORMS, POL, J4>(kr, knorm, n_chunks, TILE, te, (TILE) > tb, CUR, NXT, RKC, RKN, lds_rq[rtl],     \
                                lds_x[rtl], qf, sacc, sprev, hs, b, t0, T, chunk_enc, wave, lane, rk4, voff, voff4)
  for (int64_t tile = tb; tile < te; tile += 2) {
    MSA_RING_SUB(0, tile, ring0, ring3, rk0, rk1);
    MSA_RING_SUB(1, tile, ring1, ring0, rk0, rk1);
    if (tile + 1 < te) {
      MSA_RING_SUB(2, tile + 1, ring2, ring1, rk1, rk0);
      MSA_RING_SUB(3, tile + 1, ring3, ring2, rk1, rk0);
    }
  }
#undef MSA_RING_SUB
  // finish the last tile (the first head group receives)
  const int64_t last = te - 1;
  lds_barrier();
  if (hs == 0) {
    f32x4_t* x = lds_x[rtl] + lane;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4_t o = x[q4 * 64];
      sprev[4 * q4] += o[0]; sprev[4 * q4 + 1] += o[1]; sprev[4 * q4 + 2] += o[2]; sprev[4 * q4 + 3] += o[3];
    }
    finish_tile(sprev, half, m, t0, T, b, last, n_chunks, 1.0f / 8, chunk_enc);
  }
  wait_vmem_all();                            // the last copies land before the LDS is released
}

// ------------------------------------------------------ stored key norms
// 1/|Krbar[g, h]| for every chunk and head, fp32 [n_chunks, H].  Built once per
// routing-key store (offline, beside the store) so the online scan needs no
// norm pass of its own.  16 lanes share one 256-byte (chunk, head) row: each
// reads 16 contiguous bytes (the wave reads 1 KB contiguous), then the 16
// partial sums are added across the lanes.
__global__ void __launch_bounds__(256)
krbar_norms_kernel(const uint16_t* __restrict__ Krbar, int64_t n_rows, float* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = t >> 4;
  const int piece = (int)(t & 15);
  float ss = 0.f;
  if (r < n_rows) ss = sq_norm_piece(reinterpret_cast<const uint4*>(Krbar + r * D)[piece], 0.f);
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) ss += __shfl_xor(ss, m);
  if (r < n_rows && piece == 0) out[r] = inv_norm_fast(ss);
}

}  // namespace

// Compute units of the calling thread's current device, looked up once per device.
// Every thread that fills a slot stores the same value, so relaxed atomics suffice.
int num_cus() {
  constexpr int MAXDEV = 64;
  static int cus[MAXDEV] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev >= MAXDEV) {
    int v = 0;
    return hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0 ? v : 256;
  }
  int c = __atomic_load_n(&cus[dev], __ATOMIC_RELAXED);
  if (c == 0) {
    int v = 0;
    c = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0 ? v : 256;
    __atomic_store_n(&cus[dev], c, __ATOMIC_RELAXED);
  }
  return c;
}

namespace {

template <int H>
int launch_route_h(const uint16_t* Qr, int B, int T, const uint16_t* Krbar, const float* inv_norm,
                   int64_t n_chunks, uint32_t* chunk_enc, hipStream_t stream) {
  const int cus = num_cus();
  const int RTq = (T + RW - 1) / RW;
  const int P = (B * RTq + NW - 1) / NW;
  const int64_t n_tiles = (n_chunks + TC - 1) / TC;
  int64_t S = (cus + P - 1) / P;
  S = ((S + 7) / 8) * 8;
  if (S > n_tiles) S = n_tiles;
  if (S < 1) S = 1;
  const int64_t per = (n_tiles + S - 1) / S;
  S = (n_tiles + per - 1) / per;
  const int64_t grid = ((S + 7) / 8) * 8 * (int64_t)P;
  // The chunk maxima arrive armed: every word holds 0, the encoding's minimum (below
  // every float), so atomicMax takes the first value; the document max re-arms them.
  // A slice read by one row block is streamed once: its copies take the non-temporal
  // policy.  Several row blocks of a slice share its lines in L2, so those keep the default.
#define MSA_ROUTE_MFMA(NORMS_, POL_, KN_)                                                                    \
  do {                                                                                                       \
    if (H == 8 && B * RTq % NW == 0)                                                                         \
      hipLaunchKernelGGL((route_ring8_kernel<NORMS_, POL_>), dim3((unsigned)grid), dim3(512), 0, stream,      \
                         Qr, B, T, RTq, P, (int)S, Krbar, KN_, n_chunks, per, chunk_enc);                     \
    else                                                                                                     \
      hipLaunchKernelGGL((route_mfma_kernel<H, NORMS_, POL_>), dim3((unsigned)grid), dim3(Cfg<H>::THREADS), 0, \
                         stream, Qr, B, T, RTq, P, (int)S, Krbar, KN_, n_chunks, per, chunk_enc);             \
  } while (0)
  const bool stream_once = P == 1;
  bool launched = false;
  if constexpr (H >= 4) {
    if (inv_norm) {
      if (stream_once) MSA_ROUTE_MFMA(true, POL_NT, inv_norm);
      else MSA_ROUTE_MFMA(true, 0, inv_norm);
      launched = true;
    }
  }
  if (!launched) {
    if (stream_once) MSA_ROUTE_MFMA(false, POL_NT, (const float*)nullptr);
    else MSA_ROUTE_MFMA(false, 0, (const float*)nullptr);
  }
#undef MSA_ROUTE_MFMA
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

}  // namespace

size_t route_workspace(int B, int T, int H, int64_t n_chunks, int64_t n_docs) {
  (void)T; (void)H; (void)n_docs;
  return ((size_t)B * (size_t)n_chunks * sizeof(uint32_t) + 255) & ~(size_t)255;
}

int launch_krbar_norms(const uint16_t* Krbar, int64_t n_chunks, int H, float* inv_norm, hipStream_t stream) {
  const int64_t rows = n_chunks * H;
  if (rows == 0) return MSA_OK;
  hipLaunchKernelGGL(krbar_norms_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, stream, Krbar,
                     rows, inv_norm);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

int launch_route_scan(const uint16_t* Qr, int B, int T, int H, const uint16_t* Krbar, const float* inv_norm,
                      int64_t n_chunks, uint32_t* chunk_enc, hipStream_t stream) {
  if (n_chunks == 0) return MSA_OK;
  switch (H) {
    case 1: return launch_route_h<1>(Qr, B, T, Krbar, inv_norm, n_chunks, chunk_enc, stream);
    case 2: return launch_route_h<2>(Qr, B, T, Krbar, inv_norm, n_chunks, chunk_enc, stream);
    case 4: return launch_route_h<4>(Qr, B, T, Krbar, inv_norm, n_chunks, chunk_enc, stream);
    case 8: return launch_route_h<8>(Qr, B, T, Krbar, inv_norm, n_chunks, chunk_enc, stream);
    default: set_error("H=%d unsupported", H); return MSA_ERR_UNSUPPORTED;
  }
}

int launch_route(const uint16_t* Qr, int B, int T, int H, const uint16_t* Krbar, const float* inv_norm,
                 int64_t n_chunks, const int64_t* doc_chunk_off, int64_t n_docs, const uint8_t* doc_exclude,
                 float* doc_scores, float* chunk_scores, void* workspace, hipStream_t stream) {
  uint32_t* chunk_enc = reinterpret_cast<uint32_t*>(workspace);
  const int rc = launch_route_scan(Qr, B, T, H, Krbar, inv_norm, n_chunks, chunk_enc, stream);
  if (rc != MSA_OK) return rc;
  return launch_doc_reduce(chunk_enc, n_chunks, doc_chunk_off, n_docs, doc_exclude, B, doc_scores, chunk_scores,
                           stream);
}

int launch_clear_u32(void* p, int64_t words, hipStream_t stream) {
  if (words <= 0) return MSA_OK;
  int64_t blocks = ((words >> 2) + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(p),
                     words, 0u);
  MSA_CHECK_LAUNCH();
  return MSA_OK;
}

}  // namespace msa
