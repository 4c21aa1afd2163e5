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
hipError_t launch_gemm_large<DDG_BITS>(const GemmArgs& a, hipStream_t stream) {
  gemm_large_kernel<DDG_BITS><<<dim3((unsigned)(a.tiles_m * a.tiles_n)), dim3(512), 0, stream>>>(a);
  return hipGetLastError();
}

template <>
hipError_t launch_gemm_n192<DDG_BITS>(const GemmArgs& a, hipStream_t stream) {
  gemm_n192_kernel<DDG_BITS><<<dim3((unsigned)(a.tiles_m * a.tiles_n)), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

template <>
hipError_t launch_gemm_streamk<DDG_BITS>(const GemmArgs& a, const StreamK& sk, int grid, hipStream_t stream) {
  gemm_streamk_kernel<DDG_BITS><<<dim3((unsigned)grid), dim3(512), 0, stream>>>(a, sk);
  return hipGetLastError();
}

template <>
hipError_t launch_gemm_small<DDG_BITS>(const GemmArgs& a, int rb, int nc, int nk,
                                       hipStream_t stream) {
  const dim3 grid((unsigned)((a.n + 16 * nc - 1) / (16 * nc)));
#define DDG_SMALL(RB, NC, NK)                                                             \
  if (rb == RB && nc == NC && nk == NK) {                                                 \
    gemm_small_kernel<DDG_BITS, RB, NC, NK><<<grid, dim3(64 * NC * NK), 0, stream>>>(a); \
    return hipGetLastError();                                                             \
  }
  DDG_SMALL(1, 2, 2) DDG_SMALL(1, 1, 4) DDG_SMALL(1, 1, 8) DDG_SMALL(1, 2, 4) DDG_SMALL(1, 4, 2)
  DDG_SMALL(2, 1, 4) DDG_SMALL(2, 2, 2)
  DDG_SMALL(4, 1, 4) DDG_SMALL(4, 2, 2)
#undef DDG_SMALL
  return hipErrorInvalidValue;
}

template <>
hipError_t launch_gemm_small_split<DDG_BITS>(const GemmArgs& a, int nc, const SmallSplit& sp,
                                             hipStream_t stream) {
  if (sp.parts < 2 || sp.parts > kSmallMaxParts || nc != 2) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.n + 16 * nc - 1) / (16 * nc) * sp.parts));
  gemm_small_split_kernel<DDG_BITS, 2><<<grid, dim3(128), 0, stream>>>(a, sp);
  return hipGetLastError();
}

template <>
hipError_t launch_gemm_skinny<DDG_BITS>(const GemmArgs& a, int kc, int ncb, hipStream_t stream) {
  const dim3 grid((unsigned)((a.n + 16 * ncb - 1) / (16 * ncb)));
  if (skinny_static_lds(DDG_BITS, kc, ncb) + skinny_scale_lds(kc) > kLdsLimit) return hipErrorInvalidValue;
#define DDG_SKINNY(KC, NCB)                                                       \
  if (kc == KC && ncb == NCB) {                                                   \
    gemm_skinny_kernel<DDG_BITS, KC, NCB><<<grid, dim3(512), 0, stream>>>(a);    \
    return hipGetLastError();                                                     \
  }
  DDG_SKINNY(3, 1) DDG_SKINNY(3, 2) DDG_SKINNY(3, 4)
  DDG_SKINNY(4, 1) DDG_SKINNY(4, 2) DDG_SKINNY(4, 4)
  DDG_SKINNY(5, 1) DDG_SKINNY(5, 2) DDG_SKINNY(5, 4)
#undef DDG_SKINNY
  return hipErrorInvalidValue;
}

}  // namespace ddg
