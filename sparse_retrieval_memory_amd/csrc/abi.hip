// C ABI entry points of libmsa: host-side argument validation, then the
// launchers in the kernel sources.  Nothing is launched when validation fails.
#include "msa_internal.h"
#include "attn_split.h"

#include <string.h>

namespace msa {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }

}  // namespace msa

using msa::aligned16;

extern "C" {

int msa_version(void) { return MSA_VERSION; }

const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARG: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported shape";
    case MSA_ERR_WORKSPACE: return "workspace too small";
    case MSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* msa_last_error(void) { return msa::g_err; }

int msa_pool_chunks(const uint16_t* K, const uint16_t* V, const uint16_t* Kr, const int64_t* doc_tok_off,
                    const int64_t* doc_chunk_off, int64_t n_docs, int64_t n_tok, int64_t n_chunks, int H,
                    int D, int chunk_len, double rope_base, uint16_t* Kbar, uint16_t* Vbar,
                    uint16_t* Krbar, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(n_docs >= 1 && n_tok >= 0 && n_chunks >= 0, "n_docs >= 1, n_tok >= 0, n_chunks >= 0 required");
  MSA_CHECK_ARG(doc_tok_off && doc_chunk_off, "null offset array");
  MSA_CHECK_ARG(n_chunks == 0 || (K && V && Kr && Kbar && Vbar && Krbar), "null tensor pointer");
  MSA_CHECK_ARG(chunk_len >= 1 && chunk_len <= 1024, "chunk_len must be in [1, 1024]");
  MSA_CHECK_ARG(rope_base > 1.0, "rope_base must be > 1");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_SUPPORTED(H == 1 || H == 2 || H == 4 || H == 8 || H == 16, "H=%d unsupported", H);
  MSA_CHECK_ARG(n_chunks <= 0x7FFFFFFF, "n_chunks must fit a grid dimension");
  MSA_CHECK_ARG(n_chunks == 0 || (aligned16(K) && aligned16(V) && aligned16(Kr) && aligned16(Kbar) &&
                                  aligned16(Vbar) && aligned16(Krbar)),
                "tensor pointers must be 16-byte aligned");
  return msa::launch_pool(K, V, Kr, doc_tok_off, doc_chunk_off, n_docs, n_tok, n_chunks, H, chunk_len,
                          rope_base, Kbar, Vbar, Krbar, stream);
}

size_t msa_encode_workspace_bytes(int64_t n_chunks, int d_model) {
  if (n_chunks < 0 || d_model < 1) return 0;
  return msa::encode_workspace(n_chunks, d_model);
}

int msa_encode_router_keys(const uint16_t* hidden, int64_t n_tok, int d_model, const uint16_t* W, int H, int D,
                           const int64_t* doc_tok_off, const int64_t* doc_chunk_off, int64_t n_docs,
                           int64_t n_chunks, int chunk_len, uint16_t* Krbar, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(n_docs >= 1 && n_tok >= 0 && n_chunks >= 0, "n_docs >= 1, n_tok >= 0, n_chunks >= 0 required");
  MSA_CHECK_ARG(doc_tok_off && doc_chunk_off, "null offset array");
  MSA_CHECK_ARG(n_chunks == 0 || (hidden && W && Krbar), "null tensor pointer");
  MSA_CHECK_ARG(chunk_len >= 1 && chunk_len <= 1024, "chunk_len must be in [1, 1024]");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_SUPPORTED(H == 1 || H == 2 || H == 4 || H == 8 || H == 16, "H=%d unsupported", H);
  MSA_CHECK_SUPPORTED(d_model >= 32 && d_model <= 8192 && d_model % 32 == 0,
                      "d_model=%d unsupported (a multiple of 32 in [32, 8192])", d_model);
  MSA_CHECK_ARG(n_chunks <= 0x7FFFFFFF && n_chunks * (int64_t)d_model < ((int64_t)1 << 40), "size out of range");
  const size_t need = msa::encode_workspace(n_chunks, d_model);
  if (n_chunks > 0 && (workspace == nullptr || workspace_bytes < need)) {
    msa::set_error("workspace %zu bytes < required %zu", workspace_bytes, need);
    return MSA_ERR_WORKSPACE;
  }
  MSA_CHECK_ARG(n_chunks == 0 || (aligned16(hidden) && aligned16(W) && aligned16(Krbar) && aligned16(workspace)),
                "tensor and workspace pointers must be 16-byte aligned");
  return msa::launch_encode(hidden, n_tok, d_model, W, H * D, doc_tok_off, doc_chunk_off, n_docs, n_chunks,
                            chunk_len, Krbar, workspace, stream);
}

namespace {
// [a, a + na) and [b, b + nb) (bytes) share no byte
bool disjoint(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x + na <= y || y + nb <= x;
}
}  // namespace

size_t msa_store_delete_workspace_bytes(int64_t n_docs) {
  if (n_docs < 1) return 0;
  return msa::store_delete_workspace(n_docs);
}

int msa_store_delete(const uint16_t* Krbar, const float* inv_norm, const int64_t* doc_chunk_off, int64_t n_docs,
                     int64_t n_chunks, int H, int D, const uint8_t* keep, uint16_t* Krbar_out, float* inv_norm_out,
                     int64_t* doc_chunk_off_out, int32_t* new_id, int64_t* counts, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(n_docs >= 1 && n_docs < ((int64_t)1 << 31) && n_chunks >= 0, "1 <= n_docs < 2^31, n_chunks >= 0");
  MSA_CHECK_ARG(doc_chunk_off && keep && doc_chunk_off_out && new_id && counts, "null pointer");
  MSA_CHECK_ARG(n_chunks == 0 || (Krbar && Krbar_out), "null store pointer");
  MSA_CHECK_ARG((inv_norm == nullptr) == (inv_norm_out == nullptr), "inv_norm and inv_norm_out: both or neither");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_SUPPORTED(H == 1 || H == 2 || H == 4 || H == 8 || H == 16, "H=%d unsupported", H);
  const size_t rb = (size_t)n_chunks * H * D * 2, nbytes = (size_t)n_chunks * H * 4;
  MSA_CHECK_ARG(n_chunks == 0 || disjoint(Krbar, rb, Krbar_out, rb), "Krbar_out must not overlap Krbar");
  MSA_CHECK_ARG(!inv_norm || n_chunks == 0 || disjoint(inv_norm, nbytes, inv_norm_out, nbytes),
                "inv_norm_out must not overlap inv_norm");
  MSA_CHECK_ARG(n_chunks == 0 || (aligned16(Krbar) && aligned16(Krbar_out)), "store pointers must be 16-byte aligned");
  const size_t need = msa::store_delete_workspace(n_docs);
  if (workspace == nullptr || workspace_bytes < need) {
    msa::set_error("workspace %zu bytes < required %zu", workspace_bytes, need);
    return MSA_ERR_WORKSPACE;
  }
  MSA_CHECK_ARG(aligned16(workspace), "workspace must be 16-byte aligned");
  return msa::launch_store_delete(Krbar, inv_norm, doc_chunk_off, n_docs, H, keep, Krbar_out, inv_norm_out,
                                  doc_chunk_off_out, new_id, counts, workspace, stream);
}

int msa_store_append(uint16_t* Krbar, float* inv_norm, int64_t* doc_chunk_off, int64_t n_docs, int64_t n_chunks,
                     int H, int D, const uint16_t* new_Krbar, const int64_t* new_doc_chunk_off, int64_t n_new_docs,
                     int64_t n_new_chunks, int64_t chunk_capacity, int64_t doc_capacity, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(n_docs >= 0 && n_chunks >= 0 && n_new_docs >= 0 && n_new_chunks >= 0, "negative size");
  MSA_CHECK_ARG(doc_chunk_off && (n_new_docs == 0 || new_doc_chunk_off), "null offset array");
  MSA_CHECK_ARG(n_new_chunks == 0 || (Krbar && new_Krbar), "null store pointer");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_SUPPORTED(H == 1 || H == 2 || H == 4 || H == 8 || H == 16, "H=%d unsupported", H);
  MSA_CHECK_ARG(n_chunks + n_new_chunks <= chunk_capacity && n_docs + n_new_docs <= doc_capacity,
                "the appended store exceeds its capacity (%lld chunks, %lld documents)", (long long)chunk_capacity,
                (long long)doc_capacity);
  MSA_CHECK_ARG(n_new_chunks == 0 || (aligned16(Krbar) && aligned16(new_Krbar)), "store pointers must be 16-byte aligned");
  MSA_CHECK_ARG(n_new_chunks == 0 || disjoint(Krbar + n_chunks * (int64_t)H * D, (size_t)n_new_chunks * H * D * 2,
                                              new_Krbar, (size_t)n_new_chunks * H * D * 2),
                "new_Krbar must not overlap the store's free rows");
  return msa::launch_store_append(Krbar, inv_norm, doc_chunk_off, n_docs, n_chunks, H, new_Krbar, new_doc_chunk_off,
                                  n_new_docs, n_new_chunks, stream);
}

size_t msa_route_workspace_bytes(int B, int T, int H, int D, int64_t n_chunks, int64_t n_docs) {
  (void)D;
  if (B < 1 || T < 1 || n_chunks < 0 || n_docs < 1) return 0;
  return msa::route_workspace(B, T, H, n_chunks, n_docs);
}

int msa_krbar_inv_norms(const uint16_t* Krbar, int64_t n_chunks, int H, int D, float* inv_norm,
                        hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(n_chunks >= 0 && H >= 1, "n_chunks >= 0 and H >= 1 required");
  MSA_CHECK_ARG(n_chunks == 0 || (Krbar && inv_norm), "null pointer");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_ARG(n_chunks == 0 || aligned16(Krbar), "Krbar must be 16-byte aligned");
  MSA_CHECK_ARG(n_chunks * H < ((int64_t)1 << 38), "size out of range");
  return msa::launch_krbar_norms(Krbar, n_chunks, H, inv_norm, stream);
}

int msa_route_scores(const uint16_t* Qr, int B, int T, int H, int D, const uint16_t* Krbar,
                     const float* krbar_inv_norm, int64_t n_chunks, const int64_t* doc_chunk_off, int64_t n_docs,
                     const uint8_t* doc_exclude, float* doc_scores, float* chunk_scores, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && T >= 1, "B >= 1 and T >= 1 required (B=%d, T=%d)", B, T);
  MSA_CHECK_ARG(n_docs >= 1 && n_chunks >= 0, "n_docs >= 1 and n_chunks >= 0 required");
  MSA_CHECK_ARG(Qr && doc_chunk_off && doc_scores && (Krbar || n_chunks == 0), "null pointer");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_SUPPORTED(H == 1 || H == 2 || H == 4 || H == 8, "H=%d unsupported (1, 2, 4 or 8)", H);
  MSA_CHECK_ARG((int64_t)B * T <= (1 << 24), "B*T too large");
  MSA_CHECK_ARG(n_docs < 0x7FFFFFFF / 256 * 256 && n_chunks < ((int64_t)1 << 40), "size out of range");
  MSA_CHECK_ARG(aligned16(Qr) && (n_chunks == 0 || aligned16(Krbar)), "Qr and Krbar must be 16-byte aligned");
  const size_t need = msa::route_workspace(B, T, H, n_chunks, n_docs);
  if (workspace_bytes < need || (need > 0 && workspace == nullptr)) {
    msa::set_error("workspace %zu bytes < required %zu", workspace_bytes, need);
    return MSA_ERR_WORKSPACE;
  }
  MSA_CHECK_ARG(workspace == nullptr || aligned16(workspace), "workspace must be 16-byte aligned");
  MSA_CHECK_ARG(krbar_inv_norm == nullptr || aligned16(krbar_inv_norm), "krbar_inv_norm must be 16-byte aligned");
  return msa::launch_route(Qr, B, T, H, Krbar, krbar_inv_norm, n_chunks, doc_chunk_off, n_docs, doc_exclude,
                           doc_scores, chunk_scores, workspace, stream);
}

size_t msa_route_topk_workspace_bytes(int B, int T, int H, int D, int64_t n_chunks, int64_t n_docs, int k) {
  (void)D;
  if (B < 1 || T < 1 || n_docs < 1 || n_chunks < 0 || k < 1 || k > 32) return 0;
  const size_t r = (msa::route_workspace(B, T, H, n_chunks, n_docs) + 255) & ~(size_t)255;
  return r + msa::topk_workspace(B, n_docs, k);
}

int msa_route_topk(const uint16_t* Qr, int B, int T, int H, int D, const uint16_t* Krbar,
                   const float* krbar_inv_norm, int64_t n_chunks, const int64_t* doc_chunk_off, int64_t n_docs,
                   const uint8_t* doc_exclude, int k, float* doc_scores, float* chunk_scores, int32_t* top_idx,
                   float* top_scores, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && T >= 1, "B >= 1 and T >= 1 required (B=%d, T=%d)", B, T);
  MSA_CHECK_ARG(n_docs >= 1 && n_chunks >= 0, "n_docs >= 1 and n_chunks >= 0 required");
  MSA_CHECK_ARG(Qr && doc_chunk_off && doc_scores && top_idx && top_scores && (Krbar || n_chunks == 0),
                "null pointer");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_SUPPORTED(H == 1 || H == 2 || H == 4 || H == 8, "H=%d unsupported (1, 2, 4 or 8)", H);
  MSA_CHECK_SUPPORTED(k >= 1 && k <= 32, "k=%d unsupported here (1..32; larger k: msa_route_scores + msa_topk_docs)",
                      k);
  MSA_CHECK_ARG(k <= n_docs, "k=%d > n_docs", k);
  MSA_CHECK_ARG(B <= 65535 && (int64_t)B * T <= (1 << 24), "B*T too large");
  MSA_CHECK_ARG(n_docs < 0x7FFFFFFF / 256 * 256 && n_chunks < ((int64_t)1 << 40), "size out of range");
  MSA_CHECK_ARG(aligned16(Qr) && (n_chunks == 0 || aligned16(Krbar)), "Qr and Krbar must be 16-byte aligned");
  MSA_CHECK_ARG(krbar_inv_norm == nullptr || aligned16(krbar_inv_norm), "krbar_inv_norm must be 16-byte aligned");
  const size_t need = msa_route_topk_workspace_bytes(B, T, H, D, n_chunks, n_docs, k);
  if (workspace_bytes < need || workspace == nullptr) {
    msa::set_error("workspace %zu bytes < required %zu", workspace_bytes, need);
    return MSA_ERR_WORKSPACE;
  }
  MSA_CHECK_ARG(aligned16(workspace), "workspace must be 16-byte aligned");
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  const size_t r = (msa::route_workspace(B, T, H, n_chunks, n_docs) + 255) & ~(size_t)255;
  int rc = msa::launch_route_scan(Qr, B, T, H, Krbar, krbar_inv_norm, n_chunks, reinterpret_cast<uint32_t*>(ws),
                                  stream);
  if (rc != MSA_OK) return rc;
  return msa::launch_docs_topk(reinterpret_cast<uint32_t*>(ws), n_chunks, doc_chunk_off, n_docs, doc_exclude,
                               B, k, doc_scores, chunk_scores, top_idx, top_scores,
                               reinterpret_cast<uint64_t*>(ws + r), stream);
}

int msa_route_scan(const uint16_t* Qr, int B, int T, int H, int D, const uint16_t* Krbar,
                   const float* krbar_inv_norm, int64_t n_chunks, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && T >= 1, "B >= 1 and T >= 1 required (B=%d, T=%d)", B, T);
  MSA_CHECK_ARG(n_chunks >= 0, "n_chunks >= 0 required");
  MSA_CHECK_ARG(Qr && (Krbar || n_chunks == 0), "null pointer");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_SUPPORTED(H == 1 || H == 2 || H == 4 || H == 8, "H=%d unsupported (1, 2, 4 or 8)", H);
  MSA_CHECK_ARG(B <= 65535 && (int64_t)B * T <= (1 << 24), "B*T too large");
  MSA_CHECK_ARG(n_chunks < ((int64_t)1 << 40), "size out of range");
  MSA_CHECK_ARG(aligned16(Qr) && (n_chunks == 0 || aligned16(Krbar)), "Qr and Krbar must be 16-byte aligned");
  MSA_CHECK_ARG(krbar_inv_norm == nullptr || aligned16(krbar_inv_norm), "krbar_inv_norm must be 16-byte aligned");
  const size_t need = msa::route_workspace(B, T, H, n_chunks, 1);
  if (workspace_bytes < need || (need > 0 && workspace == nullptr)) {
    msa::set_error("workspace %zu bytes < required %zu", workspace_bytes, need);
    return MSA_ERR_WORKSPACE;
  }
  MSA_CHECK_ARG(workspace == nullptr || aligned16(workspace), "workspace must be 16-byte aligned");
  return msa::launch_route_scan(Qr, B, T, H, Krbar, krbar_inv_norm, n_chunks, reinterpret_cast<uint32_t*>(workspace),
                                stream);
}

int msa_route_select(int B, int64_t n_chunks, const int64_t* doc_chunk_off, int64_t n_docs,
                     const uint8_t* doc_exclude, int k, float* doc_scores, float* chunk_scores, int32_t* top_idx,
                     float* top_scores, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && B <= 65535, "1 <= B <= 65535 required (B=%d)", B);
  MSA_CHECK_ARG(n_docs >= 1 && n_chunks >= 0, "n_docs >= 1 and n_chunks >= 0 required");
  MSA_CHECK_ARG(doc_chunk_off && doc_scores, "null pointer");
  MSA_CHECK_SUPPORTED(k >= 0 && k <= 32, "k=%d unsupported here (0..32; larger k: msa_topk_docs)", k);
  MSA_CHECK_ARG(k <= n_docs, "k=%d > n_docs", k);
  MSA_CHECK_ARG(k == 0 || (top_idx && top_scores), "null top-k output");
  MSA_CHECK_ARG(n_docs < 0x7FFFFFFF / 256 * 256 && n_chunks < ((int64_t)1 << 40), "size out of range");
  const size_t r = (msa::route_workspace(B, 1, 1, n_chunks, n_docs) + 255) & ~(size_t)255;
  const size_t need = k == 0 ? msa::route_workspace(B, 1, 1, n_chunks, n_docs) : r + msa::topk_workspace(B, n_docs, k);
  if (workspace_bytes < need || (need > 0 && workspace == nullptr)) {
    msa::set_error("workspace %zu bytes < required %zu", workspace_bytes, need);
    return MSA_ERR_WORKSPACE;
  }
  MSA_CHECK_ARG(workspace == nullptr || aligned16(workspace), "workspace must be 16-byte aligned");
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  if (k == 0)
    return msa::launch_doc_reduce(reinterpret_cast<uint32_t*>(ws), n_chunks, doc_chunk_off, n_docs, doc_exclude, B,
                                  doc_scores, chunk_scores, stream);
  return msa::launch_docs_topk(reinterpret_cast<uint32_t*>(ws), n_chunks, doc_chunk_off, n_docs, doc_exclude, B, k,
                               doc_scores, chunk_scores, top_idx, top_scores, reinterpret_cast<uint64_t*>(ws + r),
                               stream);
}

int msa_route_workspace_clear(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(workspace != nullptr || workspace_bytes == 0, "null workspace");
  MSA_CHECK_ARG(workspace_bytes % 4 == 0, "workspace_bytes must be a multiple of 4");
  MSA_CHECK_ARG(workspace == nullptr || aligned16(workspace), "workspace must be 16-byte aligned");
  return msa::launch_clear_u32(workspace, (int64_t)(workspace_bytes / 4), stream);
}

size_t msa_route_backward_workspace_bytes(int B, int T, int H, int D, int64_t n_docs) {
  (void)D;
  if (B < 1 || T < 1 || H < 1 || n_docs < 1) return 0;
  return msa::route_bwd_workspace(B, T, H, n_docs);
}

int msa_route_scores_backward(const uint16_t* Qr, int B, int T, int H, int D, const uint16_t* Krbar,
                              const float* krbar_inv_norm, int64_t n_chunks, const int64_t* doc_chunk_off,
                              int64_t n_docs, const uint8_t* doc_exclude, const float* chunk_scores,
                              const float* d_doc_scores, float* dQr, float* dKsel, int32_t* sel, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && T >= 1, "B >= 1 and T >= 1 required (B=%d, T=%d)", B, T);
  MSA_CHECK_ARG(n_docs >= 1 && n_chunks >= 0, "n_docs >= 1 and n_chunks >= 0 required");
  MSA_CHECK_ARG(Qr && doc_chunk_off && chunk_scores && d_doc_scores && dQr && dKsel && sel &&
                    (Krbar || n_chunks == 0),
                "null pointer");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_SUPPORTED(H == 1 || H == 2 || H == 4 || H == 8, "H=%d unsupported (1, 2, 4 or 8)", H);
  MSA_CHECK_SUPPORTED(T <= msa::ROUTE_BWD_MAX_T, "T=%d unsupported (T <= %d)", T, msa::ROUTE_BWD_MAX_T);
  MSA_CHECK_ARG(B <= 65535, "B must be <= 65535");
  MSA_CHECK_ARG(n_docs < ((int64_t)1 << 30) && n_chunks < ((int64_t)1 << 40), "size out of range");
  MSA_CHECK_ARG(aligned16(Qr) && (n_chunks == 0 || aligned16(Krbar)) && aligned16(dQr) && aligned16(dKsel) &&
                    aligned16(sel),
                "Qr, Krbar, dQr, dKsel and sel must be 16-byte aligned");
  const size_t need = msa::route_bwd_workspace(B, T, H, n_docs);
  if (workspace_bytes < need || workspace == nullptr) {
    msa::set_error("workspace %zu bytes < required %zu", workspace_bytes, need);
    return MSA_ERR_WORKSPACE;
  }
  MSA_CHECK_ARG(aligned16(workspace), "workspace must be 16-byte aligned");
  return msa::launch_route_bwd(Qr, B, T, H, Krbar, krbar_inv_norm, n_chunks, doc_chunk_off, n_docs, doc_exclude,
                               chunk_scores, d_doc_scores, dQr, dKsel, sel, workspace, stream);
}

size_t msa_topk_workspace_bytes(int B, int64_t n_docs, int k) {
  if (B < 1 || n_docs < 1 || k < 1) return 0;
  return msa::topk_workspace(B, n_docs, k);
}

int msa_topk_docs(const float* doc_scores, int B, int64_t n_docs, int k, int32_t* top_idx, float* top_scores,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && n_docs >= 1, "B >= 1 and n_docs >= 1 required");
  MSA_CHECK_ARG(k >= 1 && k <= n_docs, "k=%d must satisfy 1 <= k <= n_docs (%lld)", k, (long long)n_docs);
  MSA_CHECK_ARG(n_docs < 0x7FFFFFFF, "n_docs must be < 2^31");
  MSA_CHECK_ARG(B <= 65535, "B must be <= 65535");
  MSA_CHECK_ARG(doc_scores && top_idx && top_scores, "null pointer");
  MSA_CHECK_SUPPORTED(k <= 1024, "k=%d unsupported (k <= 1024)", k);
  const size_t need = msa::topk_workspace(B, n_docs, k);
  if (workspace_bytes < need || workspace == nullptr) {
    msa::set_error("workspace %zu bytes < required %zu", workspace_bytes, need);
    return MSA_ERR_WORKSPACE;
  }
  MSA_CHECK_ARG(aligned16(workspace), "workspace must be 16-byte aligned");
  return msa::launch_topk(doc_scores, B, n_docs, k, top_idx, top_scores, workspace, stream);
}

int msa_fetch_docs(const int32_t* top_idx_host, int B, int k, const uint16_t* host_store,
                   const int64_t* doc_chunk_off_host, int64_t n_docs, int H, int D, uint16_t* staging, int Mmax,
                   int32_t* mem_len_host, hipStream_t side, hipEvent_t done) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && k >= 1 && n_docs >= 1 && Mmax >= 1 && H >= 1, "B, k, n_docs, Mmax, H must be >= 1");
  MSA_CHECK_ARG(top_idx_host && host_store && doc_chunk_off_host && staging && mem_len_host, "null pointer");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  const int64_t entry = 2LL * H * D;              // elements per staged entry
  // validate everything before the first copy
  for (int b = 0; b < B; ++b) {
    int64_t m = 0;
    for (int r = 0; r < k; ++r) {
      const int32_t d = top_idx_host[(int64_t)b * k + r];
      MSA_CHECK_ARG(d >= 0 && d < n_docs, "top_idx[%d,%d]=%d out of range", b, r, d);
      const int64_t n = doc_chunk_off_host[d + 1] - doc_chunk_off_host[d];
      MSA_CHECK_ARG(n >= 1, "document %d has no chunks", d);
      m += n;
    }
    MSA_CHECK_ARG(m <= Mmax, "query %d needs %lld entries > Mmax=%d", b, (long long)m, Mmax);
    mem_len_host[b] = (int32_t)m;
  }
  for (int b = 0; b < B; ++b) {
    int64_t m = 0;
    int r = 0;
    while (r < k) {
      // merge runs of documents whose chunks are adjacent in the store
      const int32_t d = top_idx_host[(int64_t)b * k + r];
      const int64_t g0 = doc_chunk_off_host[d];
      int64_t g1 = doc_chunk_off_host[d + 1];
      int r2 = r + 1;
      while (r2 < k && doc_chunk_off_host[top_idx_host[(int64_t)b * k + r2]] == g1) {
        g1 = doc_chunk_off_host[top_idx_host[(int64_t)b * k + r2] + 1];
        ++r2;
      }
      const size_t bytes = (size_t)((g1 - g0) * entry) * sizeof(uint16_t);
      MSA_CHECK_HIP(hipMemcpyAsync(staging + ((int64_t)b * Mmax + m) * entry, host_store + g0 * entry, bytes,
                                   hipMemcpyHostToDevice, side));
      m += g1 - g0;
      r = r2;
    }
  }
  if (done) MSA_CHECK_HIP(hipEventRecord(done, side));
  return MSA_OK;
}

int msa_gather_docs(const int32_t* top_idx, int B, int k, const uint16_t* host_store, const int64_t* doc_chunk_off,
                    int64_t n_docs, int H, int D, uint16_t* staging, int Mmax, int32_t* mem_len,
                    hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && B <= 65535 && k >= 1 && n_docs >= 1 && Mmax >= 1 && H >= 1, "bad sizes");
  MSA_CHECK_ARG(top_idx && host_store && doc_chunk_off && staging && mem_len, "null pointer");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_ARG(aligned16(host_store) && aligned16(staging), "host_store and staging must be 16-byte aligned");
  return msa::launch_gather(top_idx, B, k, host_store, doc_chunk_off, n_docs, H, staging, Mmax, mem_len, stream);
}

int msa_append_router_rows(const uint16_t* Qr, int B, int T0, int H, int D, const uint16_t* Krbar,
                           const int64_t* doc_chunk_off, int64_t n_docs, const int32_t* ids, int n_ids, int T_out,
                           uint16_t* rows, int32_t* n_rows, uint8_t* doc_exclude, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && B <= 65535 && T0 >= 1 && H >= 1 && n_docs >= 1 && n_ids >= 0, "bad sizes");
  MSA_CHECK_ARG(T_out >= T0 && T_out <= (1 << 24), "need T0 <= T_out <= 2^24");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_ARG(Qr && Krbar && doc_chunk_off && rows && (n_ids == 0 || ids), "null pointer");
  MSA_CHECK_ARG(aligned16(Qr) && aligned16(Krbar) && aligned16(rows), "Qr, Krbar and rows must be 16-byte aligned");
  return msa::launch_append_rows(Qr, B, T0, H, Krbar, doc_chunk_off, n_docs, ids, n_ids, T_out, rows, n_rows,
                                 doc_exclude, stream);
}

int msa_sparse_attn_decode(const uint16_t* Q, int B, int Tq, int Hq, int D, const uint16_t* Kloc,
                           const uint16_t* Vloc, int Tl, int Hkv, const uint16_t* Kmem, const uint16_t* Vmem,
                           int64_t mem_entry_stride, int Mmax, const int32_t* mem_len, int rope_offset,
                           double rope_base, float scale, float* O, hipStream_t stream) {
  return msa_sparse_attn_forward(Q, B, Tq, Hq, D, Kloc, Vloc, Tl, Hkv, Kmem, Vmem, mem_entry_stride, Mmax, mem_len,
                                 rope_offset, rope_base, scale, O, nullptr, stream);
}

int msa_sparse_attn_forward(const uint16_t* Q, int B, int Tq, int Hq, int D, const uint16_t* Kloc,
                            const uint16_t* Vloc, int Tl, int Hkv, const uint16_t* Kmem, const uint16_t* Vmem,
                            int64_t mem_entry_stride, int Mmax, const int32_t* mem_len, int rope_offset,
                            double rope_base, float scale, float* O, float* lse, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && B <= 65535 && Tq >= 1 && Tl >= Tq, "need B >= 1, 1 <= Tq <= Tl");
  MSA_CHECK_ARG(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0 && Hq <= 65535, "need Hq %% Hkv == 0");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_SUPPORTED(Hkv <= 16, "Hkv=%d unsupported (<= 16)", Hkv);
  MSA_CHECK_ARG(Mmax >= 0 && rope_offset >= 0 && rope_base > 1.0, "need Mmax >= 0, rope_offset >= 0, base > 1");
  MSA_CHECK_ARG(Q && Kloc && Vloc && O && mem_len, "null pointer");
  MSA_CHECK_ARG(((uintptr_t)lse & 3) == 0, "lse must be 4-byte aligned");
  MSA_CHECK_ARG(Mmax == 0 || (Kmem && Vmem && mem_entry_stride >= (int64_t)Hkv * D && mem_entry_stride % 8 == 0),
                "memory pointers/stride invalid");
  MSA_CHECK_ARG(aligned16(Q) && aligned16(Kloc) && aligned16(Vloc) && aligned16(O) &&
                    (Mmax == 0 || (aligned16(Kmem) && aligned16(Vmem))),
                "pointers must be 16-byte aligned");
  return msa::launch_attn(Q, B, Tq, Hq, Kloc, Vloc, Tl, Hkv, Kmem, Vmem, mem_entry_stride, Mmax, mem_len,
                          rope_offset, rope_base, scale, O, lse, stream);
}

int msa_sparse_attn_local_partial(const uint16_t* Q, int B, int Tq, int Hq, int D, const uint16_t* Kloc,
                                  const uint16_t* Vloc, int Tl, int Hkv, int rope_offset, double rope_base,
                                  float scale, float* part_O, float* part_ml, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && B <= 65535 && Tq >= 1 && Tl >= Tq, "need B >= 1, 1 <= Tq <= Tl");
  MSA_CHECK_ARG(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0 && Hq <= 65535, "need Hq %% Hkv == 0");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_SUPPORTED(Hkv <= 16, "Hkv=%d unsupported (<= 16)", Hkv);
  MSA_CHECK_ARG(rope_offset >= 0 && rope_base > 1.0, "need rope_offset >= 0, base > 1");
  MSA_CHECK_ARG(Q && Kloc && Vloc && part_O && part_ml, "null pointer");
  MSA_CHECK_ARG(aligned16(Q) && aligned16(Kloc) && aligned16(Vloc) && aligned16(part_O) &&
                    ((uintptr_t)part_ml & 7) == 0,
                "Q, Kloc, Vloc, part_O must be 16-byte aligned, part_ml 8-byte");
  return msa::launch_attn_local(Q, B, Tq, Hq, Kloc, Vloc, Tl, Hkv, rope_offset, rope_base, scale, part_O, part_ml,
                                stream);
}

int msa_sparse_attn_memory_merge(const uint16_t* Q, int B, int Tq, int Hq, int D, int Tl, int Hkv,
                                 const uint16_t* Kmem, const uint16_t* Vmem, int64_t mem_entry_stride, int Mmax,
                                 const int32_t* mem_len, int rope_offset, double rope_base, float scale,
                                 const float* part_O, const float* part_ml, float* O, float* lse,
                                 hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && B <= 65535 && Tq >= 1 && Tl >= Tq, "need B >= 1, 1 <= Tq <= Tl");
  MSA_CHECK_ARG(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0 && Hq <= 65535, "need Hq %% Hkv == 0");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_SUPPORTED(Hkv <= 16, "Hkv=%d unsupported (<= 16)", Hkv);
  MSA_CHECK_ARG(Mmax >= 0 && rope_offset >= 0 && rope_base > 1.0, "need Mmax >= 0, rope_offset >= 0, base > 1");
  MSA_CHECK_ARG(Q && O && mem_len && part_O && part_ml, "null pointer");
  MSA_CHECK_ARG(Mmax == 0 || (Kmem && Vmem && mem_entry_stride >= (int64_t)Hkv * D && mem_entry_stride % 8 == 0),
                "memory pointers/stride invalid");
  MSA_CHECK_ARG(aligned16(Q) && aligned16(O) && aligned16(part_O) && ((uintptr_t)part_ml & 7) == 0 &&
                    ((uintptr_t)lse & 3) == 0 && (Mmax == 0 || (aligned16(Kmem) && aligned16(Vmem))),
                "pointers misaligned (16 bytes; part_ml 8, lse 4)");
  return msa::launch_attn_memory(Q, B, Tq, Hq, Tl, Hkv, Kmem, Vmem, mem_entry_stride, Mmax, mem_len, rope_offset,
                                 rope_base, scale, part_O, part_ml, O, lse, stream);
}

size_t msa_sparse_attn_backward_workspace_bytes(int B, int Tq, int Hq, int D, int Tl, int Hkv, int Mmax) {
  (void)D;
  if (B < 1 || Tq < 1 || Tl < Tq || Hq < 1 || Hkv < 1 || Mmax < 0) return 0;
  return msa::attn_bwd_workspace(B, Tq, Hq, Tl, Hkv, Mmax);
}

int msa_sparse_attn_backward(const uint16_t* Q, int B, int Tq, int Hq, int D, const uint16_t* Kloc,
                             const uint16_t* Vloc, int Tl, int Hkv, const uint16_t* Kmem, const uint16_t* Vmem,
                             int64_t mem_entry_stride, int Mmax, const int32_t* mem_len, int rope_offset,
                             double rope_base, float scale, const float* dO, float* dQ, float* dKloc, float* dVloc,
                             float* dKmem, float* dVmem, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  return msa_sparse_attn_backward_saved(Q, B, Tq, Hq, D, Kloc, Vloc, Tl, Hkv, Kmem, Vmem, mem_entry_stride, Mmax,
                                        mem_len, rope_offset, rope_base, scale, dO, nullptr, nullptr, dQ, dKloc, dVloc,
                                        dKmem, dVmem, workspace, workspace_bytes, stream);
}

int msa_sparse_attn_backward_saved(const uint16_t* Q, int B, int Tq, int Hq, int D, const uint16_t* Kloc,
                                   const uint16_t* Vloc, int Tl, int Hkv, const uint16_t* Kmem, const uint16_t* Vmem,
                                   int64_t mem_entry_stride, int Mmax, const int32_t* mem_len, int rope_offset,
                                   double rope_base, float scale, const float* dO, const float* O, const float* lse,
                                   float* dQ, float* dKloc, float* dVloc, float* dKmem, float* dVmem, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  msa::clear_error();
  MSA_CHECK_ARG(B >= 1 && B <= 65535 && Tq >= 1 && Tl >= Tq, "need B >= 1, 1 <= Tq <= Tl");
  MSA_CHECK_ARG(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0 && Hq <= 65535, "need Hq %% Hkv == 0");
  MSA_CHECK_SUPPORTED(D == 128, "D=%d unsupported (D must be 128)", D);
  MSA_CHECK_SUPPORTED(Hkv <= 16, "Hkv=%d unsupported (<= 16)", Hkv);
  MSA_CHECK_ARG(Mmax >= 0 && rope_offset >= 0 && rope_base > 1.0, "need Mmax >= 0, rope_offset >= 0, base > 1");
  MSA_CHECK_ARG((int64_t)Mmax + Tl < (1 << 24) && Tq < (1 << 24), "sizes out of range");
  MSA_CHECK_ARG(Q && Kloc && Vloc && mem_len && dO && dQ && dKloc && dVloc, "null pointer");
  MSA_CHECK_ARG(Mmax == 0 || (Kmem && Vmem && dKmem && dVmem && mem_entry_stride >= (int64_t)Hkv * D &&
                               mem_entry_stride % 8 == 0),
                "memory pointers/stride invalid");
  MSA_CHECK_ARG(aligned16(Q) && aligned16(Kloc) && aligned16(Vloc) && aligned16(dO) && aligned16(dQ) &&
                    aligned16(dKloc) && aligned16(dVloc) &&
                    (Mmax == 0 || (aligned16(Kmem) && aligned16(Vmem) && aligned16(dKmem) && aligned16(dVmem))),
                "pointers must be 16-byte aligned");
  MSA_CHECK_ARG((O == nullptr) == (lse == nullptr), "O and lse are given together or not at all");
  MSA_CHECK_ARG(O == nullptr || (aligned16(O) && ((uintptr_t)lse & 3) == 0), "O must be 16-byte aligned, lse 4-byte");
  const size_t need = msa::attn_bwd_workspace(B, Tq, Hq, Tl, Hkv, Mmax);
  if (workspace_bytes < need || workspace == nullptr) {
    msa::set_error("workspace %zu bytes < required %zu", workspace_bytes, need);
    return MSA_ERR_WORKSPACE;
  }
  MSA_CHECK_ARG(aligned16(workspace), "workspace must be 16-byte aligned");
  return msa::launch_attn_bwd(Q, B, Tq, Hq, Kloc, Vloc, Tl, Hkv, Kmem, Vmem, mem_entry_stride, Mmax, mem_len,
                              rope_offset, rope_base, scale, dO, O, lse, dQ, dKloc, dVloc, dKmem, dVmem, workspace,
                              stream);
}

}  // extern "C"
