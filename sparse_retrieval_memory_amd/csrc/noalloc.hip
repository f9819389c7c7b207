// msa_route_topk_noalloc: msa_route_topk with its workspace in a fixed device array
// of the library, for callers that cannot allocate (code under graph capture,
// serving loops, harnesses that forbid allocation).
//
// The array lives in this file as a static device symbol; host code never uses
// its name as an address: the first call on a device (with that device current)
// asks the runtime for the device address once, keeps it per device, and clears
// the array with a kernel.  Every later call leaves it zeroed (the routing
// calls hand their workspace back cleared), so it is cleared again only after a
// call that failed while launching.  Calls that overlap on one device race on
// the array.
#include "msa_internal.h"

#include <mutex>

namespace msa {

static __device__ __align__(256) uint8_t scratch[MSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAXDEV = 64;
struct DevScratch {
  void* ptr;
  bool clean;      // zero, as the routing calls expect on entry
};
DevScratch g_dev[MAXDEV] = {};
std::mutex g_mu;

}  // namespace
}  // namespace msa

extern "C" int msa_route_topk_noalloc(const uint16_t* Qr, int B, int T, int H, int D, const uint16_t* Krbar,
                                      const float* krbar_inv_norm, int64_t n_chunks, const int64_t* doc_chunk_off,
                                      int64_t n_docs, const uint8_t* doc_exclude, int k, float* doc_scores,
                                      float* chunk_scores, int32_t* top_idx, float* top_scores, hipStream_t stream) {
  // validate every argument first, with nothing touched on the device: msa_route_topk without a
  // workspace checks them all and, for a valid call, stops at the missing workspace
  const int vrc = msa_route_topk(Qr, B, T, H, D, Krbar, krbar_inv_norm, n_chunks, doc_chunk_off, n_docs, doc_exclude,
                                 k, doc_scores, chunk_scores, top_idx, top_scores, nullptr, 0, stream);
  if (vrc != MSA_ERR_WORKSPACE) return vrc;
  msa::clear_error();
  const size_t need = msa_route_topk_workspace_bytes(B, T, H, D, n_chunks, n_docs, k);
  if (need > (size_t)MSA_NOALLOC_SCRATCH_BYTES) {
    msa::set_error("needs %zu bytes of scratch, more than the fixed %zu (B * n_chunks * 4 + B * ceil(n_docs / 64) * 8 "
                   "must fit)", need, (size_t)MSA_NOALLOC_SCRATCH_BYTES);
    return MSA_ERR_WORKSPACE;
  }
  int dev = 0;
  MSA_CHECK_HIP(hipGetDevice(&dev));
  MSA_CHECK_ARG(dev >= 0 && dev < msa::MAXDEV, "device %d beyond the %d this entry point supports", dev, msa::MAXDEV);
  void* ws = nullptr;
  bool clean = false;
  {
    std::lock_guard<std::mutex> lk(msa::g_mu);
    if (msa::g_dev[dev].ptr == nullptr) {
      void* p = nullptr;
      MSA_CHECK_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(msa::scratch)));
      msa::g_dev[dev].ptr = p;
      msa::g_dev[dev].clean = false;
    }
    ws = msa::g_dev[dev].ptr;
    clean = msa::g_dev[dev].clean;
  }
  if (!clean) {
    const int rc = msa::launch_clear_u32(ws, (int64_t)(MSA_NOALLOC_SCRATCH_BYTES / 4), stream);
    if (rc != MSA_OK) return rc;
  }
  const int rc = msa_route_topk(Qr, B, T, H, D, Krbar, krbar_inv_norm, n_chunks, doc_chunk_off, n_docs, doc_exclude,
                                k, doc_scores, chunk_scores, top_idx, top_scores, ws, need, stream);
  {
    std::lock_guard<std::mutex> lk(msa::g_mu);
    // a call rejected before launching leaves the array as it was; a launch failure may leave it dirty
    if (rc == MSA_OK) msa::g_dev[dev].clean = true;
    else if (rc == MSA_ERR_HIP) msa::g_dev[dev].clean = false;
    else msa::g_dev[dev].clean = clean;
  }
  return rc;
}
