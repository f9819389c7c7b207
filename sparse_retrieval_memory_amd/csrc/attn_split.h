// Launchers of the split sparse attention (the local-key partial and the memory pass that
// merges with it); defined in attn.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {
int launch_attn_local(const uint16_t* Q, int B, int Tq, int Hq, const uint16_t* Kloc, const uint16_t* Vloc, int Tl,
                      int Hkv, int rope_offset, double rope_base, float scale, float* part_O, float* part_ml,
                      hipStream_t stream);
int launch_attn_memory(const uint16_t* Q, int B, int Tq, int Hq, int Tl, int Hkv, const uint16_t* Kmem,
                       const uint16_t* Vmem, int64_t mem_entry_stride, int Mmax, const int32_t* mem_len,
                       int rope_offset, double rope_base, float scale, const float* part_O, const float* part_ml,
                       float* O, float* lse, hipStream_t stream);
}  // namespace msa
