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
// a.tiles_m / a.tiles_n: 256 x 256 tiles
template <int B>
hipError_t launch_gemm_large(const GemmArgs& a, hipStream_t stream);
// a.tiles_m / a.tiles_n: 256 x 192 tiles
template <int B>
hipError_t launch_gemm_n192(const GemmArgs& a, hipStream_t stream);
// rb: row blocks (of 16) in 1, 2, 4; nc column waves x nk K-split waves per
// workgroup: (2,2) (1,4) (1,8) (2,4) (4,2) for rb = 1, (1,4) (2,2) otherwise
template <int B>
hipError_t launch_gemm_small(const GemmArgs& a, int rb, int nc, int nk, hipStream_t stream);
// split-K or stream-K over a.tiles_m x a.tiles_n tiles of 256 x 256 with
// `grid` workgroups (sk.split x tiles, or 8 sk.wpx); sk.partials / sk.flags:
// workspace of `grid` slots
template <int B>
hipError_t launch_gemm_streamk(const GemmArgs& a, const StreamK& sk, int grid, hipStream_t stream);

// M <= 16 with K split across workgroups: nc (2) column blocks of 16 per
// workgroup, sp.parts parts of K (grid ceil(n / 16 nc) x parts)
template <int B>
hipError_t launch_gemm_small_split(const GemmArgs& a, int nc, const SmallSplit& sp, hipStream_t stream);

template <int B>
hipError_t launch_gemm_skinny(const GemmArgs& a, int kc, int ncb, hipStream_t stream);

// up to kMaxGroup products with M <= 16 in one launch of ga.ncb (1, 2 or 4)
// column blocks of 16 per workgroup (ga.wg_start is the prefix sum of
// ceil(n / (16 ga.ncb)) over the products)
hipError_t launch_gemm_grouped(const GroupArgs& ga, hipStream_t stream);
// up to kMaxGroup products with M > 64 in one launch of 256 x 256 tiles
// (ga.tile_start is the prefix sum of the products' tile counts)
hipError_t launch_gemm_grouped_large(const GroupLargeArgs& ga, hipStream_t stream);
// up to kMaxGroup products with 16 < M <= 16 rb (rb = 2 or 4) in one launch
// (ga.wg_start is the prefix sum of ceil(n / 32) over the products)
hipError_t launch_gemm_grouped_small(const GroupArgs& ga, int rb, hipStream_t stream);

// per-row and total quantization error at widths 3..7 (row_sse: n x 5)
hipError_t launch_quant_sse(const void* w, bool f32_in, int64_t n, int64_t k, double* row_sse,
                            double* total, hipStream_t stream);

// RPBH rotation of n rows of d (d % 64 == 0, d % h == 0, d <= kRotateMaxD,
// h a power of two in 2..1024)
constexpr int kRotateMaxD = 16384;
hipError_t launch_rpbh_rotate(const void* x, bool f32_in, int64_t n, int d, const int32_t* perm,
                              const int8_t* signs, int h, void* out, bool f32_out, int cus,
                              hipStream_t stream);

// FP4 weights x FP8 activations (formats: kFp4E2M1, kFp4E3M0, kFp4E1M2)
constexpr int kFp4E2M1 = 0, kFp4E3M0 = 1, kFp4E1M2 = 2;
struct W4A8Args {
  const uint8_t* xq;        // M x K E4M3 codes
  const float* xscales;     // M per-token scales
  const uint8_t* packed;    // N x K/2 bytes of 4-bit codes
  const float* wscales;     // N x K/128 group scales
  void* y;                  // M x N
  int m, n, k;
  int tiles_m, tiles_n;     // set by the launcher (its tile shape)
  int out_bf16;
};
// pow2: group scales rounded up to powers of two, applied by the matrix
// instructions as their block scales; tiled: codes and scales in 32-column
// blocks, in the order the matrix operands load them
hipError_t launch_fp4_quantize_pack(const void* w, bool f32_in, int64_t n, int k, int fmt, bool pow2, bool tiled,
                                    uint32_t* packed, float* scales, hipStream_t stream);
hipError_t launch_fp8_quantize_rows(const uint16_t* x, int64_t m, int k, uint8_t* q, float* sx,
                                    hipStream_t stream);
hipError_t launch_w4a8_gemm(const W4A8Args& a, int fmt, bool pow2, bool tiled, hipStream_t stream);
// 6-bit activations (formats kFp6E2M3, kFp6E3M2) in the tiled 6-bit storage;
// the product takes tiled FP4 weights of format fmt (xq of W4A8Args: the
// 6-bit storage)
constexpr int kFp6E2M3 = 0, kFp6E3M2 = 1;
hipError_t launch_fp6_quantize_rows(const uint16_t* x, int64_t m, int k, int fmt6, uint8_t* q, float* sx,
                                    hipStream_t stream);
hipError_t launch_w4a6_gemm(const W4A8Args& a, int fmt, int fmt6, bool pow2, hipStream_t stream);
// FP6 weights (kFp6E2M3, kFp6E3M2) per group of 128 in the tiled 6-bit
// storage (weight rows in place of tokens) with tiled scales, and their
// product with E4M3 activations (xq, xscales of W4A8Args)
constexpr int kFp6wE2M3 = 3, kFp6wE3M2 = 4;   // weight formats of the product kernel
hipError_t launch_fp6w_quantize_pack(const void* w, bool f32_in, int64_t n, int k, int fmt6, bool pow2,
                                     uint8_t* packed, float* scales, hipStream_t stream);
hipError_t launch_w6a8_gemm(const W4A8Args& a, int fmt6, bool pow2, hipStream_t stream);

hipError_t launch_lowrank_t(const __bf16* x, const __bf16* lora_down, __bf16* t, int m, int k,
                            int r, hipStream_t stream);
// K chunks of the split pre-pass for k inputs (whole groups, at most 32
// chunks): gpc groups per chunk; returns the chunk count.
int lowrank_split_chunks(int k, int* gpc);
// The split pre-pass: float32 partials (chunks x m x r) in part, then T.
hipError_t launch_lowrank_t_split(const __bf16* x, const __bf16* lora_down, __bf16* t, float* part,
                                  int m, int k, int r, hipStream_t stream);

}  // namespace ddg
