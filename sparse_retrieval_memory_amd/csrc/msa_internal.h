// Internal helpers shared by the HIP sources of libmsa (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/msa.h"

namespace msa {

// ------------------------------------------------------------ error reporting
void set_error(const char* fmt, ...);
void clear_error();

#define MSA_CHECK_ARG(cond, ...)                 \
  do {                                           \
    if (!(cond)) {                               \
      ::msa::set_error(__VA_ARGS__);             \
      return MSA_ERR_INVALID_ARG;                \
    }                                            \
  } while (0)

#define MSA_CHECK_SUPPORTED(cond, ...)           \
  do {                                           \
    if (!(cond)) {                               \
      ::msa::set_error(__VA_ARGS__);             \
      return MSA_ERR_UNSUPPORTED;                \
    }                                            \
  } while (0)

#define MSA_CHECK_HIP(expr)                                                   \
  do {                                                                        \
    hipError_t e_ = (expr);                                                   \
    if (e_ != hipSuccess) {                                                   \
      ::msa::set_error("%s failed: %s", #expr, hipGetErrorString(e_));        \
      return MSA_ERR_HIP;                                                     \
    }                                                                         \
  } while (0)

#define MSA_CHECK_LAUNCH()                                                    \
  do {                                                                        \
    hipError_t e_ = hipGetLastError();                                        \
    if (e_ != hipSuccess) {                                                   \
      ::msa::set_error("kernel launch failed: %s", hipGetErrorString(e_));    \
      return MSA_ERR_HIP;                                                     \
    }                                                                         \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------------ device helpers
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// two fp32 -> packed bf16 pair (a in the low half), gfx950's packed conversion
// instruction (round to nearest even)
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// RoPE: cos/sin of pos * theta_i, theta_i = base^(-2i/D), given rev_i = theta_i / (2 pi)
// in fp64.  The angle in revolutions is reduced to [-1/2, 1/2] in fp64, then
// evaluated in fp32.
__device__ __forceinline__ void rope_cs(int pos, double rev_i, float* c, float* s) {
  double r = (double)pos * rev_i;
  r -= rint(r);
  sincospif(2.0f * (float)r, s, c);
}

// Order-preserving map float -> uint32 (a < b  <=>  enc(a) < enc(b) for non-NaN).
__device__ __forceinline__ uint32_t enc_f32(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float dec_f32(uint32_t e) {
  uint32_t u = (e & 0x80000000u) ? (e & 0x7FFFFFFFu) : ~e;
  return __uint_as_float(u);
}

// sum of a*b over two packed bf16 pairs, fp32 accumulate
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// LDS-only barrier: wait for this wave's LDS traffic, then s_barrier.  Unlike
// __syncthreads() it does not wait for outstanding global loads, so LDS-DMA
// prefetches stay in flight across it.  The waits use the builtin (gfx9
// encoding) so the compiler's own wait-count tracking sees them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt/expcnt untouched
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Wait until every vector-memory operation issued by this wave has completed.
__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  asm volatile("" ::: "memory");
}

// Inclusive scan of (a, b) over a workgroup of up to 1024 threads (a multiple
// of 64): shuffles within each wave, then the wave totals.  s_a / s_b: LDS
// scratch of blockDim.x / 64 entries; callers barrier before reusing them.
__device__ __forceinline__ void block_scan2(int64_t& a, int64_t& b, int64_t* s_a, int64_t* s_b) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int64_t ua = __shfl_up(a, s), ub = __shfl_up(b, s);
    if (lane >= s) { a += ua; b += ub; }
  }
  if (lane == 63) { s_a[wave] = a; s_b[wave] = b; }
  __syncthreads();
  int64_t ba = 0, bb = 0;
  for (int w = 0; w < wave; ++w) { ba += s_a[w]; bb += s_b[w]; }
  a += ba;
  b += bb;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Asynchronous 16-byte-per-lane global -> LDS copy.  The LDS destination of
// lane i is lds_base + 16 * i (lds_base must be wave-uniform).
// POL is the copy's cache policy: 0 = default, POL_NT = non-temporal (streamed data
// that no other workgroup re-reads; on MI355X a stream of such copies reaches ~7.1 TB/s
// against ~6.3 TB/s with the default policy).
constexpr int POL_NT = 2;
template <int POL = 0>
__device__ __forceinline__ void dma16(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void_t*)lds_base, 16, 0, POL);
}

// 16-byte vector load with the non-temporal policy, for data a kernel reads once.
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

}  // namespace msa

// kernel-family launchers (defined in the .hip files)
namespace msa {
int launch_pool(const uint16_t* K, const uint16_t* V, const uint16_t* Kr, const int64_t* doc_tok_off,
                const int64_t* doc_chunk_off, int64_t n_docs, int64_t n_tok, int64_t n_chunks, int H,
                int chunk_len, double rope_base, uint16_t* Kbar, uint16_t* Vbar, uint16_t* Krbar,
                hipStream_t stream);
// Routing workspace contract: the chunk maxima (B * n_chunks uint32, the order-preserving
// encoding) start at 0 and are set back to 0 by the document max that reads them; the
// top-k's group maxima are cleared by the selection that reads them.
int launch_route(const uint16_t* Qr, int B, int T, int H, const uint16_t* Krbar, const float* inv_norm,
                 int64_t n_chunks, const int64_t* doc_chunk_off, int64_t n_docs, const uint8_t* doc_exclude,
                 float* doc_scores, float* chunk_scores, void* workspace, hipStream_t stream);
int launch_route_scan(const uint16_t* Qr, int B, int T, int H, const uint16_t* Krbar, const float* inv_norm,
                      int64_t n_chunks, uint32_t* chunk_enc, hipStream_t stream);
// Compute units of the calling thread's current device (looked up once per device).
int num_cus();
int launch_doc_reduce(uint32_t* chunk_enc, int64_t n_chunks, const int64_t* doc_chunk_off, int64_t n_docs,
                      const uint8_t* doc_exclude, int B, float* doc_scores, float* chunk_scores, hipStream_t stream);
int launch_clear_u32(void* p, int64_t words, hipStream_t stream);
int launch_krbar_norms(const uint16_t* Krbar, int64_t n_chunks, int H, float* inv_norm, hipStream_t stream);
size_t route_workspace(int B, int T, int H, int64_t n_chunks, int64_t n_docs);
int launch_topk(const float* doc_scores, int B, int64_t n_docs, int k, int32_t* top_idx,
                float* top_scores, void* workspace, hipStream_t stream);
size_t topk_workspace(int B, int64_t n_docs, int k);
// Document max from the scan's chunk maxima fused with top-k's group maxima, then the
// group-based top-k (1 <= k <= 32); gmax holds B * ceil(n_docs / 64) keys.
int launch_docs_topk(uint32_t* chunk_enc, int64_t n_chunks, const int64_t* doc_chunk_off, int64_t n_docs,
                     const uint8_t* doc_exclude, int B, int k, float* doc_scores, float* chunk_scores,
                     int32_t* top_idx, float* top_scores, uint64_t* gmax, hipStream_t stream);
int launch_attn(const uint16_t* Q, int B, int Tq, int Hq, const uint16_t* Kloc, const uint16_t* Vloc,
                int Tl, int Hkv, const uint16_t* Kmem, const uint16_t* Vmem, int64_t mem_entry_stride,
                int Mmax, const int32_t* mem_len, int rope_offset, double rope_base, float scale,
                float* O, float* lse, hipStream_t stream);
int launch_attn_bwd(const uint16_t* Q, int B, int Tq, int Hq, const uint16_t* Kloc, const uint16_t* Vloc, int Tl,
                    int Hkv, const uint16_t* Kmem, const uint16_t* Vmem, int64_t mem_entry_stride, int Mmax,
                    const int32_t* mem_len, int rope_offset, double rope_base, float scale, const float* dO,
                    const float* O, const float* lse, float* dQ, float* dKloc, float* dVloc, float* dKmem,
                    float* dVmem, void* workspace, hipStream_t stream);
size_t attn_bwd_workspace(int B, int Tq, int Hq, int Tl, int Hkv, int Mmax);
int launch_append_rows(const uint16_t* Qr, int B, int T0, int H, const uint16_t* Krbar,
                       const int64_t* doc_chunk_off, int64_t n_docs, const int32_t* ids, int n_ids, int T_out,
                       uint16_t* rows, int32_t* n_rows, uint8_t* doc_exclude, hipStream_t stream);
int launch_encode(const uint16_t* hidden, int64_t n_tok, int dm, const uint16_t* W, int N,
                  const int64_t* doc_tok_off, const int64_t* doc_chunk_off, int64_t n_docs, int64_t n_chunks,
                  int chunk_len, uint16_t* Krbar, void* workspace, hipStream_t stream);
size_t encode_workspace(int64_t n_chunks, int dm);
int launch_store_delete(const uint16_t* rows, const float* norms, const int64_t* off, int64_t n_docs, int H,
                        const uint8_t* keep, uint16_t* rows_out, float* norms_out, int64_t* off_out,
                        int32_t* new_id, int64_t* counts, void* workspace, hipStream_t stream);
size_t store_delete_workspace(int64_t n_docs);
int launch_route_bwd(const uint16_t* Qr, int B, int T, int H, const uint16_t* Krbar, const float* inv_norm,
                     int64_t n_chunks, const int64_t* doc_chunk_off, int64_t n_docs, const uint8_t* doc_exclude,
                     const float* chunk_scores, const float* d_doc_scores, float* dQr, float* dKsel, int32_t* sel,
                     void* workspace, hipStream_t stream);
size_t route_bwd_workspace(int B, int T, int H, int64_t n_docs);
constexpr int ROUTE_BWD_MAX_T = 8192;
int launch_store_append(uint16_t* rows, float* norms, int64_t* off, int64_t n_docs, int64_t n_chunks, int H,
                        const uint16_t* new_rows, const int64_t* new_off, int64_t n_new_docs, int64_t n_new_chunks,
                        hipStream_t stream);
int launch_gather(const int32_t* top_idx, int B, int k, const uint16_t* host_store,
                  const int64_t* doc_chunk_off, int64_t n_docs, int H, uint16_t* staging, int Mmax,
                  int32_t* mem_len, hipStream_t stream);
}  // namespace msa
