/*
 * msa.h -- C ABI of the Memory Sparse Attention (MSA) routing + sparse-attention
 * hot path for AMD Instinct MI355X (gfx950).
 *
 * The calls follow the three-stage inference pipeline the MSA pages describe
 * (b-lab.team summary of MSA, "Global Memory Encoding", "Online Routing &
 * Context Assembly", "Sparse Generation"):
 *
 *   msa_pool_chunks         offline: chunk-mean pooled (Kbar, Vbar, Krbar) cache
 *   msa_encode_router_keys  offline: router keys projected from hidden states, chunk-mean pooled
 *   msa_store_delete        update: delete documents from the routing store (compacted copy)
 *   msa_store_append        update: append documents to the routing store in place
 *   msa_krbar_inv_norms     offline: 1/|Krbar| per chunk and head, stored beside the store
 *   msa_route_scores        online: cosine routing scan over every Krbar chunk
 *   msa_route_scan, msa_route_select  the same as two calls: the scan, then document max + top-k
 *   msa_route_scores_backward  training: gradient of the routing scores (Qr, selected Krbar)
 *   msa_topk_docs           online: the k most relevant documents
 *   msa_fetch_docs          online: copy the selected content KV from pinned host
 *   msa_gather_docs         online: same, as one device kernel reading mapped host memory
 *   msa_append_router_rows  interleave: the next round's router rows and exclusions
 *   msa_sparse_attn_decode  generation: GQA attention over [memory ++ local KV]
 *   msa_route_topk             msa_route_scores + msa_topk_docs in one call (k <= 32)
 *   msa_route_topk_noalloc     the same with a fixed scratch array in the library (no workspace)
 *   msa_sparse_attn_local_partial, msa_sparse_attn_memory_merge  the same attention in two launches
 *                              (the local-key half needs nothing retrieved)
 *   msa_sparse_attn_forward    training: the same attention, also returning each row's log-sum-exp
 *   msa_sparse_attn_backward   training: gradient of that attention (Q, local K/V, memory K/V)
 *   msa_sparse_attn_backward_saved  the same gradient from the forward's saved output and log-sum-exp
 *
 * Conventions (every call):
 *   - Tensors are row-major with the last dimension contiguous.  bf16 tensors
 *     are passed as uint16_t bit patterns.  Pointers are device pointers
 *     unless the parameter name ends in _host.
 *   - The caller allocates and frees every buffer (including workspaces and the
 *     pinned host store).  The library allocates nothing.  Its only state: a
 *     thread-local error message; per host thread, the RoPE constants of the
 *     last attention launch (a pure function of its rope_offset and rope_base,
 *     kept to skip recomputing them); per device, the compute-unit count (read
 *     once, used to size the routing scan's grid) and the address of the
 *     fixed-size scratch array that msa_route_topk_noalloc uses in place of a
 *     workspace (a static device array of the library, present from load).
 *   - Calls are asynchronous on `stream`; results are valid once the stream has
 *     reached the call.  Arguments are validated on the host before anything
 *     is launched: an invalid call returns a negative status and launches
 *     nothing.  HIP launch errors return MSA_ERR_HIP.  msa_last_error() gives
 *     a human-readable reason for the last failure on the calling thread.
 *   - Device pointers must be 16-byte aligned.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_OK 0
#define MSA_ERR_INVALID_ARG (-1)   /* null pointer, bad size, bad alignment, ... */
#define MSA_ERR_UNSUPPORTED (-2)   /* a shape the library does not implement (e.g. D != 128) */
#define MSA_ERR_WORKSPACE (-3)     /* workspace smaller than the *_workspace_bytes() value */
#define MSA_ERR_HIP (-4)           /* a HIP runtime call failed */

#define MSA_VERSION 100            /* 1.0.0 */

int msa_version(void);
const char* msa_status_string(int status);
/* Reason for the most recent failing call on this thread ("" if none). */
const char* msa_last_error(void);

/*
 * msa_pool_chunks -- chunk-mean pooling of one routed layer (offline encoding).
 *
 * Defined by: medium write-up sec. 2 and b-lab.team summary sec. 1 (documents
 * are cut into fixed-length chunks and K, V and the router key K_r are
 * mean-pooled per chunk); b-lab.team sec. 1, Document-wise RoPE (positions
 * restart at 0 in every document).
 *
 * For document d with L_d = doc_tok_off[d+1] - doc_tok_off[d] tokens and chunk
 * j covering local tokens [j*chunk_len, min((j+1)*chunk_len, L_d)), chunk
 * g = doc_chunk_off[d] + j gets
 *   Kbar[g]  = mean_t RoPE(K[t], t_local)     (pairs (i, i+D/2), angle t_local*base^(-2i/D))
 *   Vbar[g]  = mean_t V[t]
 *   Krbar[g] = mean_t Kr[t]
 * accumulated in fp32 (angles in fp64) and rounded to bf16 (nearest even).
 * A trailing partial chunk is averaged over its actual length.
 *
 *   K, V, Kr            bf16 [n_tok, H, D]          tokens of the documents, in order
 *   doc_tok_off         int64 [n_docs+1] (device)   token offsets; doc_tok_off[0] may be
 *                                                    non-zero (slab processing): token t of
 *                                                    the corpus is row t - doc_tok_off[0]
 *   doc_chunk_off       int64 [n_docs+1] (device)   chunk offsets, doc_chunk_off[d+1] -
 *                                                    doc_chunk_off[d] = ceil(L_d/chunk_len) >= 1;
 *                                                    output row = chunk - doc_chunk_off[0]
 *   n_tok, n_chunks     rows of the inputs / outputs (used for validation and bounds)
 *   H in {1,2,4,8,16}, D == 128, chunk_len in [1, 1024]
 *   Kbar, Vbar, Krbar   bf16 [n_chunks, H, D] outputs
 */
int msa_pool_chunks(const uint16_t* K, const uint16_t* V, const uint16_t* Kr,
                    const int64_t* doc_tok_off, const int64_t* doc_chunk_off, int64_t n_docs,
                    int64_t n_tok, int64_t n_chunks, int H, int D, int chunk_len,
                    double rope_base, uint16_t* Kbar, uint16_t* Vbar, uint16_t* Krbar,
                    hipStream_t stream);

/*
 * msa_encode_router_keys -- router keys of a corpus from its hidden states
 * (offline encoding, the step that produces Krbar).
 *
 * Defined by: b-lab.team summary, pipeline stage "Global Memory Encoding" (a
 * forward pass over the corpus caches chunk-pooled K_r) and sec. 1 (a router
 * projector maps hidden states to the routing space; the router keys are
 * chunk-mean pooled like K and V).  Reading: K_r,t = hidden[t] W^T, no bias.
 *
 * With chunks as in msa_pool_chunks (same offsets, a trailing partial chunk
 * averaged over its actual length):
 *   Krbar[g, h, :] = mean_{t in chunk g} (hidden[t] W^T)[h*D : (h+1)*D]
 * computed as the projection of the chunk's mean hidden state (the same value
 * in exact arithmetic): the mean is summed in fp32 and carried as a bf16 hi+lo
 * pair (~2^-17 relative), the products are exact bf16 products accumulated in
 * fp32, and the result is rounded to bf16 (nearest even).
 *
 *   hidden       bf16 [n_tok, d_model]        hidden states of the documents, in order
 *   W            bf16 [H*D, d_model]          router-key projection (out x in)
 *   doc_tok_off, doc_chunk_off, n_docs, n_tok, n_chunks, chunk_len: as in msa_pool_chunks
 *   Krbar        bf16 [n_chunks, H, D] out
 *   workspace    >= msa_encode_workspace_bytes(n_chunks, d_model) bytes (the chunk means)
 *   d_model a multiple of 32 in [32, 8192]; H in {1,2,4,8,16}; D == 128; chunk_len in [1, 1024]
 */
size_t msa_encode_workspace_bytes(int64_t n_chunks, int d_model);
int msa_encode_router_keys(const uint16_t* hidden, int64_t n_tok, int d_model, const uint16_t* W, int H,
                           int D, const int64_t* doc_tok_off, const int64_t* doc_chunk_off, int64_t n_docs,
                           int64_t n_chunks, int chunk_len, uint16_t* Krbar, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * msa_store_delete / msa_store_append -- incremental updates of the routing store.
 *
 * Defined by: chatpaper.ai page, Abstract (an inability to modify memory content
 * dynamically is listed among the alternatives' weaknesses).  Reading: deleted
 * documents disappear; survivors keep their order, are renumbered 0, 1, ... and
 * move with all their chunk rows; appended documents follow the last one.  Rows
 * are moved, not recomputed: an updated store is bit-identical to one built from
 * the same documents from scratch.  (The pinned host content tier is the
 * caller's to compact with the same new_id map.)
 *
 * msa_store_delete (out of place):
 *   Krbar          bf16 [n_chunks, H, D]   store; n_chunks == doc_chunk_off[n_docs]
 *   inv_norm       fp32 [n_chunks, H] or NULL (then inv_norm_out must be NULL too)
 *   doc_chunk_off  int64 [n_docs+1] (device), doc_chunk_off[0] == 0
 *   keep           uint8 [n_docs] (device): nonzero = keep
 *   Krbar_out      bf16 [<= n_chunks, H, D], inv_norm_out fp32 [<= n_chunks, H]:
 *                  the survivors' rows; must not overlap Krbar / inv_norm
 *   doc_chunk_off_out int64 [n_docs+1] capacity: the survivors' offsets
 *   new_id         int32 [n_docs]: new index of each document, -1 if deleted
 *   counts         int64 [2] (device): surviving documents, surviving chunks
 *   workspace      >= msa_store_delete_workspace_bytes(n_docs) bytes
 *   1 <= n_docs < 2^31; H in {1,2,4,8,16}; D == 128
 *
 * msa_store_append (in place, within capacity):
 *   Krbar [chunk_capacity, H, D], inv_norm [chunk_capacity, H] or NULL (then the
 *   appended chunks' inverse norms are not computed), doc_chunk_off
 *   [doc_capacity+1]: the store with n_docs documents and n_chunks ==
 *   doc_chunk_off[n_docs] chunks; new_Krbar bf16 [n_new_chunks, H, D] and
 *   new_doc_chunk_off int64 [n_new_docs+1] (device, new_doc_chunk_off[0] == 0,
 *   new_doc_chunk_off[n_new_docs] == n_new_chunks) are the documents to add.
 *   On return the store holds n_docs + n_new_docs documents.
 *   n_chunks + n_new_chunks <= chunk_capacity, n_docs + n_new_docs <= doc_capacity.
 */
size_t msa_store_delete_workspace_bytes(int64_t n_docs);
int msa_store_delete(const uint16_t* Krbar, const float* inv_norm, const int64_t* doc_chunk_off, int64_t n_docs,
                     int64_t n_chunks, int H, int D, const uint8_t* keep, uint16_t* Krbar_out, float* inv_norm_out,
                     int64_t* doc_chunk_off_out, int32_t* new_id, int64_t* counts, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);
int msa_store_append(uint16_t* Krbar, float* inv_norm, int64_t* doc_chunk_off, int64_t n_docs, int64_t n_chunks,
                     int H, int D, const uint16_t* new_Krbar, const int64_t* new_doc_chunk_off, int64_t n_new_docs,
                     int64_t n_new_chunks, int64_t chunk_capacity, int64_t doc_capacity, hipStream_t stream);

/*
 * msa_route_scores -- routing scan: chunk and document relevance.
 *
 * Defined by: b-lab.team summary sec. 1 (cosine similarity of the query's
 * router projection Q_r with the pooled K_r, averaged over heads, then the
 * token-wise maximum) and medium write-up sec. 2 (chunk similarity selects the
 * most relevant documents).
 *
 *   S[b,t,g]           = (1/H) sum_h cos(Qr[b,t,h,:], Krbar[g,h,:])   (cos := 0 on a zero vector)
 *   chunk_scores[b,g]  = max_{t<T} S[b,t,g]
 *   doc_scores[b,d]    = max over d's chunks, or -inf where doc_exclude[b,d] != 0 or
 *                        where d has no chunks (doc_chunk_off[d] == doc_chunk_off[d+1])
 *
 *   Qr            bf16 [B, T, H, D]
 *   Krbar         bf16 [n_chunks, H, D]        (HBM-resident routing-key store)
 *   krbar_inv_norm fp32 [n_chunks, H] from msa_krbar_inv_norms for this Krbar, or
 *                 NULL (the scan then derives the norms from the tiles it streams)
 *   doc_chunk_off int64 [n_docs+1] (device), non-decreasing, doc_chunk_off[0] == 0,
 *                 doc_chunk_off[n_docs] == n_chunks (empty documents allowed)
 *   doc_exclude   uint8 [B, n_docs] or NULL
 *   doc_scores    fp32 [B, n_docs] out
 *   chunk_scores  fp32 [B, n_chunks] out, or NULL
 *   workspace     >= msa_route_workspace_bytes(B, T, H, D, n_chunks, n_docs) bytes, all
 *                 zero before its first use (hipMemset, a zero-filled allocation or
 *                 msa_route_workspace_clear); every successful call returns it to zero,
 *                 so it can be reused without clearing.  After MSA_ERR_HIP clear it again.
 *   H in {1,2,4,8}, D == 128, B >= 1, T >= 1, n_docs >= 1.
 * Products use the raw bf16 operands (exact) with fp32 accumulation; norms are
 * applied in fp32.  Results are deterministic (max reductions only).
 */
size_t msa_route_workspace_bytes(int B, int T, int H, int D, int64_t n_chunks, int64_t n_docs);
int msa_route_scores(const uint16_t* Qr, int B, int T, int H, int D,
                     const uint16_t* Krbar, const float* krbar_inv_norm, int64_t n_chunks,
                     const int64_t* doc_chunk_off, int64_t n_docs,
                     const uint8_t* doc_exclude, float* doc_scores, float* chunk_scores,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msa_route_scores_backward -- gradient of the routing scores.
 *
 * Defined by: b-lab.team summary sec. 2 (an auxiliary routing loss supervises
 * the sparse attention during training) and chatpaper.ai Abstract (MSA is
 * trained end to end), applied to the forward of msa_route_scores.  Given
 * d_doc_scores = dL/d doc_scores it returns dL/dQr and, per (query, document),
 * dL/dKrbar of the document's selected chunk.  Each max passes its gradient to
 * its first maximiser: the selected chunk g is the lowest-index maximum of
 * chunk_scores over the document's chunks, and the selected token t the
 * lowest-index maximum of S[b, :, g] (recomputed in fp32).  Per head, with
 * q^ = q/|q|, k^ = k/|k|, c = q^.k^ and w = d_doc_scores[b,d] / H:
 *   dQr[b,t,h,:]   += w (k^ - c q^) / |q|      (k = Krbar[g,h,:], q = Qr[b,t,h,:])
 *   dKsel[b,d,h,:]  = w (q^ - c k^) / |k|
 * A document that is empty, excluded, or has d_doc_scores == 0 passes nothing
 * (sel = (-1, -1), dKsel row 0); a zero q or k passes nothing for its head.
 *
 *   Qr, Krbar, krbar_inv_norm, doc_chunk_off, doc_exclude: as given to
 *                   msa_route_scores (krbar_inv_norm may be NULL)
 *   chunk_scores    fp32 [B, n_chunks]: that call's chunk_scores output
 *   d_doc_scores    fp32 [B, n_docs]
 *   dQr             fp32 [B, T, H, D] out (every element written)
 *   dKsel           fp32 [B, n_docs, H, D] out: the gradient w.r.t. Krbar[sel[b,d,0]]
 *                   (sum over b to accumulate into a store-shaped gradient)
 *   sel             int32 [B, n_docs, 2] out: (chunk, token) or (-1, -1)
 *   workspace       >= msa_route_backward_workspace_bytes(B, T, H, D, n_docs) bytes
 *   H in {1,2,4,8}, D == 128, 1 <= T <= 8192, 1 <= B <= 65535, 1 <= n_docs < 2^30.
 * Deterministic: the query gradient is summed in document order, without atomics.
 */
size_t msa_route_backward_workspace_bytes(int B, int T, int H, int D, int64_t n_docs);
int msa_route_scores_backward(const uint16_t* Qr, int B, int T, int H, int D,
                              const uint16_t* Krbar, const float* krbar_inv_norm, int64_t n_chunks,
                              const int64_t* doc_chunk_off, int64_t n_docs, const uint8_t* doc_exclude,
                              const float* chunk_scores, const float* d_doc_scores,
                              float* dQr, float* dKsel, int32_t* sel,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msa_krbar_inv_norms -- 1/|Krbar[g, h, :]| for every pooled chunk and head.
 *
 * The cosine of msa_route_scores (b-lab.team summary sec. 1) divides by the
 * norm of each pooled router key.  The store is built once, offline (b-lab.team
 * pipeline stage 1), so its norms can be computed once beside it and streamed
 * with it (32 bytes per 2 KB chunk at H = 8) instead of being recomputed by every
 * query's scan.  Zero vectors give 0 (so their cosine is 0).
 *
 *   Krbar      bf16 [n_chunks, H, D], D == 128
 *   inv_norm   fp32 [n_chunks, H] out (hardware reciprocal square root, ~1 ulp)
 * Pass the result as krbar_inv_norm to msa_route_scores / msa_route_topk /
 * msa_route_scan (used when H >= 4; with H < 4 the scan derives the norms from
 * the tiles it streams).
 */
int msa_krbar_inv_norms(const uint16_t* Krbar, int64_t n_chunks, int H, int D, float* inv_norm,
                        hipStream_t stream);

/*
 * msa_topk_docs -- the k most relevant documents per query.
 *
 * Defined by: medium write-up sec. 2, b-lab.team sec. 1 and pipeline stage 2,
 * jkf87 blog "core technique 1: Top-k Sparse Attention".
 *
 *   doc_scores  fp32 [B, n_docs]
 *   top_idx     int32 [B, k] out: score descending, equal scores -> lower id first
 *   top_scores  fp32 [B, k] out
 *   1 <= k <= min(n_docs, 1024); n_docs < 2^31.
 *   workspace   >= msa_topk_workspace_bytes(B, n_docs, k) bytes
 */
size_t msa_topk_workspace_bytes(int B, int64_t n_docs, int k);
int msa_topk_docs(const float* doc_scores, int B, int64_t n_docs, int k,
                  int32_t* top_idx, float* top_scores,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msa_route_topk -- msa_route_scores followed by msa_topk_docs in one call, for
 * 1 <= k <= 32: the document max and the top-k's per-64-document group maxima
 * are formed in one pass over the chunk maxima (one launch fewer).
 *
 * Defined by: as msa_route_scores and msa_topk_docs (same outputs, bit for bit).
 *   arguments as msa_route_scores, plus k and
 *   top_idx     int32 [B, k] out; top_scores fp32 [B, k] out
 *   workspace   >= msa_route_topk_workspace_bytes(B, T, H, D, n_chunks, n_docs, k)
 *               bytes, 16-byte aligned (0 returned for k outside 1..32); zero before
 *               its first use and returned to zero by every successful call, as for
 *               msa_route_scores
 *   doc_scores  fp32 [B, n_docs] out (as msa_route_scores); chunk_scores optional
 */
size_t msa_route_topk_workspace_bytes(int B, int T, int H, int D, int64_t n_chunks, int64_t n_docs, int k);
int msa_route_topk(const uint16_t* Qr, int B, int T, int H, int D, const uint16_t* Krbar,
                   const float* krbar_inv_norm, int64_t n_chunks, const int64_t* doc_chunk_off, int64_t n_docs,
                   const uint8_t* doc_exclude, int k, float* doc_scores, float* chunk_scores,
                   int32_t* top_idx, float* top_scores, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * msa_route_scan / msa_route_select -- msa_route_topk (or msa_route_scores) as two
 * calls: the scan over the store (the only step whose cost grows with the memory),
 * then the document max and the top-k.  Between them the chunk maxima live in the
 * workspace (an opaque encoding), so the two calls must get the same workspace, in
 * order, on one stream (or ordered by events).  The scan alone can then be timed
 * or overlapped with other work.
 *
 * Defined by: as msa_route_scores (b-lab.team summary sec. 1, the cosine scan and
 * the token maximum) and msa_topk_docs (document selection).
 *
 * msa_route_scan:   Qr, B, T, H, D, Krbar, krbar_inv_norm, n_chunks as msa_route_scores;
 *                   workspace >= msa_route_workspace_bytes(B, T, H, D, n_chunks, 1) bytes,
 *                   zero on entry (see msa_route_scores).
 * msa_route_select: B, n_chunks, doc_chunk_off, n_docs, doc_exclude, doc_scores,
 *                   chunk_scores as msa_route_scores; 0 <= k <= 32.  k == 0: document
 *                   scores only (top_idx, top_scores may be NULL; workspace >=
 *                   msa_route_workspace_bytes); k >= 1: also top_idx int32 [B, k] and
 *                   top_scores fp32 [B, k] as msa_topk_docs, workspace >=
 *                   msa_route_topk_workspace_bytes(B, 1, 1, 128, n_chunks, n_docs, k).
 *                   Returns the workspace to zero.
 * scan + select(k) gives msa_route_topk's outputs bit for bit; scan + select(0) gives
 * msa_route_scores'.
 */
int msa_route_scan(const uint16_t* Qr, int B, int T, int H, int D, const uint16_t* Krbar,
                   const float* krbar_inv_norm, int64_t n_chunks, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);
int msa_route_select(int B, int64_t n_chunks, const int64_t* doc_chunk_off, int64_t n_docs,
                     const uint8_t* doc_exclude, int k, float* doc_scores, float* chunk_scores, int32_t* top_idx,
                     float* top_scores, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msa_route_workspace_clear -- set a routing workspace to zero with a kernel on
 * `stream` (no memset node, so it can be recorded into a graph); needed once per
 * new workspace and after a call that returned MSA_ERR_HIP.
 *   workspace_bytes a multiple of 4; workspace 16-byte aligned.
 */
int msa_route_workspace_clear(void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msa_route_topk_noalloc -- msa_route_topk without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).
 *
 * Same arguments, outputs and errors as msa_route_topk, minus the workspace: the
 * call uses a fixed array of MSA_NOALLOC_SCRATCH_BYTES (16 MiB) inside the library,
 * one per device, held until the process ends.  The call fails with
 * MSA_ERR_WORKSPACE (nothing launched) when
 *   msa_route_topk_workspace_bytes(B, T, H, D, n_chunks, n_docs, k) > MSA_NOALLOC_SCRATCH_BYTES,
 * i.e. roughly when B * n_chunks * 4 + B * ceil(n_docs / 64) * 8 exceeds 16 MiB
 * (a 100M-token store at batch 1 needs 6.7 MB).  It allocates nothing itself.  All
 * calls on one device share that device's array: calls that overlap on one device
 * (several streams or threads at once) race and must be serialised by the caller.
 * The first call on a device looks up the array's device address and clears it
 * with a kernel on `stream`; later calls find it zeroed.
 */
#define MSA_NOALLOC_SCRATCH_BYTES (16u << 20)
int msa_route_topk_noalloc(const uint16_t* Qr, int B, int T, int H, int D, const uint16_t* Krbar,
                           const float* krbar_inv_norm, int64_t n_chunks, const int64_t* doc_chunk_off,
                           int64_t n_docs, const uint8_t* doc_exclude, int k, float* doc_scores, float* chunk_scores,
                           int32_t* top_idx, float* top_scores, hipStream_t stream);

/*
 * msa_fetch_docs -- context assembly from the host tier (host-driven copies).
 *
 * Defined by: medium write-up sec. 4B and b-lab.team sec. 2 (routing keys stay
 * in GPU memory, content K/V live in host DRAM and only the selected items are
 * fetched asynchronously); b-lab.team pipeline stage 2 (load only the
 * selected Kbar/Vbar).
 *
 * For each query b, the selected documents' chunks are copied in rank order,
 * chunks in order, with one hipMemcpyAsync per run of adjacent chunks, on
 * `side`; `done` (if not NULL) is recorded on `side` after the last copy.
 *
 *   top_idx_host        int32 [B, k] (host)
 *   host_store          bf16 [n_chunks, 2, H, D] pinned host memory: entry g = (Kbar[g], Vbar[g])
 *   doc_chunk_off_host  int64 [n_docs+1] (host)
 *   staging             bf16 [B, Mmax, 2, H, D] (device) out
 *   mem_len_host        int32 [B] (host) out: entries written for each query
 * Fails with MSA_ERR_INVALID_ARG (nothing copied) if a selected id is out of
 * range or a query's chunks exceed Mmax.
 */
int msa_fetch_docs(const int32_t* top_idx_host, int B, int k,
                   const uint16_t* host_store, const int64_t* doc_chunk_off_host, int64_t n_docs,
                   int H, int D, uint16_t* staging, int Mmax, int32_t* mem_len_host,
                   hipStream_t side, hipEvent_t done);

/*
 * msa_gather_docs -- the same assembly as msa_fetch_docs, done by one kernel on
 * `stream` that reads the (mapped, pinned) host store directly, so the selected
 * ids never travel to the host.  Chunks beyond Mmax are dropped and mem_len is
 * capped at Mmax (check mem_len against the expected total if that matters).
 *
 *   top_idx        int32 [B, k] (device)
 *   host_store     pinned host memory [n_chunks, 2, H, D], device-accessible
 *   doc_chunk_off  int64 [n_docs+1] (device)
 *   staging        bf16 [B, Mmax, 2, H, D] (device) out
 *   mem_len        int32 [B] (device) out
 */
int msa_gather_docs(const int32_t* top_idx, int B, int k,
                    const uint16_t* host_store, const int64_t* doc_chunk_off, int64_t n_docs,
                    int H, int D, uint16_t* staging, int Mmax, int32_t* mem_len,
                    hipStream_t stream);

/*
 * msa_append_router_rows -- query preparation for the next Memory Interleave
 * round.
 *
 * Defined by: medium write-up sec. 4C and b-lab.team summary sec. 3 (the
 * documents retrieved in one round become part of the next round's query).
 * Reading: the next round routes with the original router rows followed by
 * the pooled router keys (all heads) of every chunk of every document
 * retrieved so far, in retrieval order, and never selects those documents
 * again.
 *
 * For each query b: rows[b, 0..T0) = Qr[b]; then, for i = 0..n_ids-1, the
 * rows Krbar[g] of document ids[b, i]'s chunks g in order; the remaining rows
 * up to T_out repeat rows[b, 0] (a repeated row changes no token max, so the
 * scores of the padded batch equal those of each query's own rows).  Rows
 * beyond T_out are dropped: size T_out = T0 + max_b (chunks of b's ids).
 *
 *   Qr             bf16 [B, T0, H, D] (device)
 *   Krbar          bf16 [n_chunks, H, D] (device)
 *   doc_chunk_off  int64 [n_docs+1] (device)
 *   ids            int32 [B, n_ids] (device); ids outside [0, n_docs) are skipped
 *   rows           bf16 [B, T_out, H, D] (device) out
 *   n_rows         int32 [B] (device) out, or NULL: T0 + the listed chunks, capped at T_out
 *   doc_exclude    uint8 [B, n_docs] (device) or NULL: set to 1 for every listed document
 * D must be 128.  Asynchronous on `stream`.
 */
int msa_append_router_rows(const uint16_t* Qr, int B, int T0, int H, int D,
                           const uint16_t* Krbar, const int64_t* doc_chunk_off, int64_t n_docs,
                           const int32_t* ids, int n_ids, int T_out,
                           uint16_t* rows, int32_t* n_rows, uint8_t* doc_exclude, hipStream_t stream);

/*
 * msa_sparse_attn_decode -- GQA attention over [pooled memory ++ causal local KV].
 *
 * Defined by: medium write-up sec. 2 and b-lab.team sec. 1 (the selected
 * documents' compressed K/V are concatenated with the query's local K/V for
 * autoregressive decoding); b-lab.team sec. 1, Global RoPE (the query's start
 * index is offset by k, the number of retrieved blocks).
 *
 * Query row i sits at position rope_offset + (Tl - Tq) + i, local key j at
 * rope_offset + j (both rotated here); memory keys are used as given (already
 * rotated at document-local positions by msa_pool_chunks).  Every memory entry
 * is visible to every row; local key j is visible to row i iff
 * j <= (Tl - Tq) + i.  q-head h reads kv-head h / (Hq / Hkv).
 *   O[b,i,h,:] = softmax_j(scale * <q_i, k_j>) . v_j
 *
 *   Q           bf16 [B, Tq, Hq, D] (unrotated)
 *   Kloc, Vloc  bf16 [B, Tl, Hkv, D] (Kloc unrotated)
 *   Kmem, Vmem  bf16, entry m of query b at ptr + (b*Mmax + m) * mem_entry_stride,
 *               each entry [Hkv, D]; the staging layout of msa_fetch_docs gives
 *               Kmem = staging, Vmem = staging + Hkv*D, mem_entry_stride = 2*Hkv*D
 *   mem_len     int32 [B] (device): entries used per query (clamped to [0, Mmax])
 *   O           fp32 [B, Tq, Hq, D] out
 *   D == 128, 1 <= Tq <= Tl, Hq % Hkv == 0, Hkv <= 16, rope_offset >= 0.
 */
int msa_sparse_attn_decode(const uint16_t* Q, int B, int Tq, int Hq, int D,
                           const uint16_t* Kloc, const uint16_t* Vloc, int Tl, int Hkv,
                           const uint16_t* Kmem, const uint16_t* Vmem,
                           int64_t mem_entry_stride, int Mmax, const int32_t* mem_len,
                           int rope_offset, double rope_base, float scale,
                           float* O, hipStream_t stream);

/*
 * msa_sparse_attn_forward -- msa_sparse_attn_decode that also returns each
 * row's log-sum-exp, for training (msa_sparse_attn_backward_saved reuses it).
 *
 * Defined by: as msa_sparse_attn_decode; the log-sum-exp is the normaliser of
 * the softmax there:
 *   lse[b,i,h] = ln sum_{visible j} exp(scale * <q_i, k_j>)   (natural log)
 *
 *   arguments as msa_sparse_attn_decode, plus
 *   lse         fp32 [B, Tq, Hq] out, 4-byte aligned; NULL skips it (then this
 *               is msa_sparse_attn_decode)
 */
int msa_sparse_attn_forward(const uint16_t* Q, int B, int Tq, int Hq, int D,
                            const uint16_t* Kloc, const uint16_t* Vloc, int Tl, int Hkv,
                            const uint16_t* Kmem, const uint16_t* Vmem,
                            int64_t mem_entry_stride, int Mmax, const int32_t* mem_len,
                            int rope_offset, double rope_base, float scale,
                            float* O, float* lse, hipStream_t stream);

/*
 * msa_sparse_attn_local_partial / msa_sparse_attn_memory_merge -- the same
 * attention as msa_sparse_attn_decode in two launches, so that the local-key
 * half can run while the memory is still being selected and assembled.
 *
 * Defined by: as msa_sparse_attn_decode.  The softmax over [memory ++ local]
 * splits exactly into two partial sums over the two key sets, each with its
 * own running maximum, combined at the end:
 *   local_partial:  m_L = max_j s_j,  l_L = sum_j 2^(s_j - m_L),
 *                   part_O = sum_j 2^(s_j - m_L) v_j      (local keys j, visible)
 *   memory_merge:   the same over the memory entries, then
 *                   O = (2^(m_M - m) sum_M + 2^(m_L - m) part_O) / (2^(m_M - m) l_M + 2^(m_L - m) l_L),
 *                   m = max(m_M, m_L)
 * with s_j = scale * log2(e) * <q_i, k_j> (log2 units).  Query positions do not
 * depend on the memory (rope_offset is the number of selected documents, known
 * before selection), so the local partial needs only Q and the local K/V.
 *
 *   Q, Kloc, Vloc, Tl, Hkv, rope_offset, rope_base, scale: as msa_sparse_attn_decode
 *   part_O      fp32 [B, Tq, Hq, D] (written by local_partial, read by memory_merge),
 *               16-byte aligned
 *   part_ml     fp32 [B, Tq, Hq, 2] = (m_L, l_L), 8-byte aligned
 *   Kmem, Vmem, mem_entry_stride, Mmax, mem_len: as msa_sparse_attn_decode
 *   O           fp32 [B, Tq, Hq, D] out; lse fp32 [B, Tq, Hq] out or NULL
 *               (natural log, as msa_sparse_attn_forward)
 * memory_merge must be ordered after local_partial on the caller's streams.
 */
int msa_sparse_attn_local_partial(const uint16_t* Q, int B, int Tq, int Hq, int D,
                                  const uint16_t* Kloc, const uint16_t* Vloc, int Tl, int Hkv,
                                  int rope_offset, double rope_base, float scale,
                                  float* part_O, float* part_ml, hipStream_t stream);
int msa_sparse_attn_memory_merge(const uint16_t* Q, int B, int Tq, int Hq, int D, int Tl, int Hkv,
                                 const uint16_t* Kmem, const uint16_t* Vmem,
                                 int64_t mem_entry_stride, int Mmax, const int32_t* mem_len,
                                 int rope_offset, double rope_base, float scale,
                                 const float* part_O, const float* part_ml,
                                 float* O, float* lse, hipStream_t stream);

/*
 * msa_sparse_attn_backward -- gradient of msa_sparse_attn_decode.
 *
 * Defined by: chatpaper.ai Abstract (MSA is trained end to end, so the loss
 * reaches the query, the local context and the retrieved memory through this
 * attention), applied to the forward of msa_sparse_attn_decode (medium
 * write-up sec. 2, b-lab.team sec. 1 and its Global RoPE bullet).  Per q-head,
 * with S = scale * Qrot Krot^T over the visible keys, P = softmax_rows(S):
 *   dV = P^T dO,  dS = P * (dO V^T - rowsum(P * dO V^T)),
 *   dQrot = scale * dS K,  dK = scale * dS^T Qrot;
 * a kv-head collects the gradients of the q-heads that read it, and the
 * gradients of Q and Kloc (rotated inside the forward) are rotated back.
 * Memory keys are used as given (already rotated by msa_pool_chunks), so dKmem
 * is the gradient of the given entries.
 *
 *   Q, Kloc, Vloc, Kmem, Vmem, mem_entry_stride, Mmax, mem_len, rope_offset,
 *   rope_base, scale: as given to msa_sparse_attn_decode
 *   dO          fp32 [B, Tq, Hq, D]
 *   dQ          fp32 [B, Tq, Hq, D] out
 *   dKloc, dVloc fp32 [B, Tl, Hkv, D] out
 *   dKmem, dVmem fp32 [B, Mmax, Hkv, D] out (dense; entries >= mem_len[b] are set to 0);
 *               may be NULL when Mmax == 0
 *   workspace   >= msa_sparse_attn_backward_workspace_bytes(B, Tq, Hq, D, Tl, Hkv, Mmax) bytes
 *   D == 128, 1 <= Tq <= Tl, Hq % Hkv == 0, Hkv <= 16, rope_offset >= 0.
 * Products use bf16 hi + lo splits of every fp32 operand with fp32 accumulation;
 * results are deterministic (no atomics).
 */
size_t msa_sparse_attn_backward_workspace_bytes(int B, int Tq, int Hq, int D, int Tl, int Hkv, int Mmax);
int msa_sparse_attn_backward(const uint16_t* Q, int B, int Tq, int Hq, int D,
                             const uint16_t* Kloc, const uint16_t* Vloc, int Tl, int Hkv,
                             const uint16_t* Kmem, const uint16_t* Vmem,
                             int64_t mem_entry_stride, int Mmax, const int32_t* mem_len,
                             int rope_offset, double rope_base, float scale,
                             const float* dO, float* dQ, float* dKloc, float* dVloc,
                             float* dKmem, float* dVmem,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msa_sparse_attn_backward_saved -- msa_sparse_attn_backward given the
 * forward's output O and log-sum-exp (msa_sparse_attn_forward), which replace
 * the pass that recomputes every row's softmax statistics:
 *   rowsum(P * dO V^T) = rowsum(dO * O),  P = exp(S - lse).
 * Same definition, arguments and outputs as msa_sparse_attn_backward, plus
 *   O           fp32 [B, Tq, Hq, D], 16-byte aligned (the forward's output)
 *   lse         fp32 [B, Tq, Hq], 4-byte aligned (its log-sum-exp)
 * Both NULL: identical to msa_sparse_attn_backward; one of them NULL: error.
 * The same workspace size applies.
 */
int msa_sparse_attn_backward_saved(const uint16_t* Q, int B, int Tq, int Hq, int D,
                                   const uint16_t* Kloc, const uint16_t* Vloc, int Tl, int Hkv,
                                   const uint16_t* Kmem, const uint16_t* Vmem,
                                   int64_t mem_entry_stride, int Mmax, const int32_t* mem_len,
                                   int rope_offset, double rope_base, float scale,
                                   const float* dO, const float* O, const float* lse,
                                   float* dQ, float* dKloc, float* dVloc,
                                   float* dKmem, float* dVmem,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
