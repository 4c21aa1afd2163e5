// Host-side launchers of the libddg kernels (one explicit instantiation per
// bit width lives in inst_bits.hip, compiled once for each B in 3..7).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ddg_kernels.hpp"

namespace ddg {

template <int B>
hipError_t launch_quantize_pack(const void* w, bool f32_in, int64_t n_chunks, uint32_t* packed,
                                float* scales, hipStream_t stream);
template <int B>
hipError_t launch_dequantize(const uint8_t* packed, const float* scales, int64_t n_chunks,
                             void* out, hipStream_t stream);
// cb: column blocks (of 16) per wave, 2 or 3
template <int B>
hipError_t launch_gemm_large(const GemmArgs& a, int cb, hipStream_t stream);
// rb: row blocks (of 16) in 1, 2, 4; cb: column blocks per workgroup in 1, 2, 4
template <int B>
hipError_t launch_gemm_small(const GemmArgs& a, int rb, int cb, hipStream_t stream);

hipError_t launch_lowrank_t(const __bf16* x, const __bf16* lora_down, __bf16* t, int m, int k,
                            int r, hipStream_t stream);

}  // namespace ddg
