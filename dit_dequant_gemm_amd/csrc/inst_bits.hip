// Kernel instantiations for one bit width, DDG_BITS (set by the build: the
// file is compiled once per width so the five widths build in parallel).
#include "ddg_launch.hpp"

#ifndef DDG_BITS
#error "compile with -DDDG_BITS=<3..7>"
#endif

namespace ddg {

namespace {
inline unsigned blocks_for(int64_t items, int per_block) {
  return (unsigned)((items + per_block - 1) / per_block);
}
}  // namespace

template <>
hipError_t launch_quantize_pack<DDG_BITS>(const void* w, bool f32_in, int64_t n_chunks,
                                          uint32_t* packed, float* scales, hipStream_t stream) {
  const dim3 grid(blocks_for(n_chunks, 256)), block(256);
  if (f32_in)
    quantize_pack_kernel<DDG_BITS, true><<<grid, block, 0, stream>>>(w, n_chunks, packed, scales);
  else
    quantize_pack_kernel<DDG_BITS, false><<<grid, block, 0, stream>>>(w, n_chunks, packed, scales);
  return hipGetLastError();
}

template <>
hipError_t launch_dequantize<DDG_BITS>(const uint8_t* packed, const float* scales,
                                       int64_t n_chunks, void* out, hipStream_t stream) {
  dequantize_kernel<DDG_BITS><<<dim3(blocks_for(n_chunks, 256)), dim3(256), 0, stream>>>(
      packed, scales, n_chunks, static_cast<u32x4*>(out));
  return hipGetLastError();
}

template <>
hipError_t launch_gemm_large<DDG_BITS>(const GemmArgs& a, int cb, hipStream_t stream) {
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(256);
  switch (cb) {
    case 2: gemm_large_kernel<DDG_BITS, 2><<<grid, block, 0, stream>>>(a); break;
    case 3: gemm_large_kernel<DDG_BITS, 3><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <>
hipError_t launch_gemm_small<DDG_BITS>(const GemmArgs& a, int rb, int cb, hipStream_t stream) {
  const dim3 grid((unsigned)((a.n + 16 * cb - 1) / (16 * cb)));
#define DDG_SMALL(RB, CB, NW)                                                          \
  if (rb == RB && cb == CB) {                                                          \
    gemm_small_kernel<DDG_BITS, RB, CB, NW><<<grid, dim3(64 * NW), 0, stream>>>(a);    \
    return hipGetLastError();                                                          \
  }
  DDG_SMALL(1, 1, 8) DDG_SMALL(1, 2, 8) DDG_SMALL(1, 4, 8)
  DDG_SMALL(2, 1, 8) DDG_SMALL(2, 2, 8) DDG_SMALL(2, 4, 8)
  DDG_SMALL(4, 1, 8) DDG_SMALL(4, 2, 8) DDG_SMALL(4, 4, 4)
#undef DDG_SMALL
  return hipErrorInvalidValue;
}

}  // namespace ddg
