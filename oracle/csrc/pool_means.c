/* Oracle (test infrastructure only): chunk means of bf16 rows in float64.
 *
 * The V / K_r part of the chunk-mean pooling the MSA pages describe (medium
 * write-up sec. 2 and b-lab.team summary sec. 1: documents are cut into
 * fixed-length chunks and each chunk is mean-pooled; a trailing partial chunk
 * is averaged over its actual length and chunks never cross documents).  The
 * same definition as oracle.msa_oracle.pool_means, in plain C so that the
 * oracle can pool a whole 10M-token corpus in seconds.  Every bf16 value is
 * exact in float64 and the sum of one chunk's values is exact as well, so the
 * result is the exact mean rounded once.  Shares nothing with the HIP path.
 */
#include <stdint.h>
#include <stdlib.h>

static inline double bf16_to_double(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)b << 16;
  return (double)v.f;
}

/* X: bf16 bits [n_tok, row] (the documents' tokens, in order); doc_len: [n_docs];
 * out: float64 [n_chunks, row]; chunk j of document d covers its tokens
 * [j*chunk, min((j+1)*chunk, L_d)).  Returns the number of chunks, -1 if out of memory. */
int64_t oracle_pool_means_bf16(const uint16_t* X, int64_t row, const int64_t* doc_len, int64_t n_docs,
                               int64_t chunk, double* out) {
  int64_t n_chunks = 0;
  for (int64_t d = 0; d < n_docs; ++d) n_chunks += (doc_len[d] + chunk - 1) / chunk;
  int64_t* first = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_chunks + 1));
  int64_t* count = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_chunks + 1));
  if (!first || !count) {
    free(first);
    free(count);
    return -1;
  }
  int64_t tok = 0, g = 0;
  for (int64_t d = 0; d < n_docs; ++d) {
    for (int64_t a = 0; a < doc_len[d]; a += chunk, ++g) {
      first[g] = tok + a;
      count[g] = doc_len[d] - a < chunk ? doc_len[d] - a : chunk;
    }
    tok += doc_len[d];
  }
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < n_chunks; ++c) {
    double* o = out + c * row;
    for (int64_t e = 0; e < row; ++e) o[e] = 0.0;
    for (int64_t t = first[c]; t < first[c] + count[c]; ++t) {
      const uint16_t* x = X + t * row;
      for (int64_t e = 0; e < row; ++e) o[e] += bf16_to_double(x[e]);
    }
    for (int64_t e = 0; e < row; ++e) o[e] /= (double)count[c];
  }
  free(first);
  free(count);
  return n_chunks;
}
