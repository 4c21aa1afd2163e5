// Launcher of the grouped small-M product (all bit widths in one kernel).
#include "ddg_launch.hpp"

namespace ddg {

template <int NCB>
__global__ __launch_bounds__(512) void gemm_grouped_skinny_kernel(GroupArgs ga) {
  using L = SkinnyLds<7, 5, NCB>;
  __shared__ __attribute__((aligned(1024))) uint8_t wl0[L::W0];
  __shared__ __attribute__((aligned(1024))) uint8_t wl1[L::W1];
  __shared__ __attribute__((aligned(256))) float scw_mem[L::NW * 5 * 64];
  const int bid = blockIdx.x;
  int j = 0;
  while (j + 1 < ga.count && bid >= ga.wg_start[j + 1]) ++j;
  j = __builtin_amdgcn_readfirstlane(j);
  const int wg = bid - ga.wg_start[j];
  const int bits = ga.bits[j], kc = ga.kc[j];
  auto run = [&]<int B, int KC>() __attribute__((always_inline)) {
    skinny_body<B, KC, NCB>(ga.g[j], wg, wl0, wl1, reinterpret_cast<float (*)[KC][64]>(scw_mem));
  };
#define DDG_GROUPED_CASE(B)                      \
  case B:                                        \
    if (kc == 3) run.template operator()<B, 3>(); \
    else if (kc == 4) run.template operator()<B, 4>(); \
    else run.template operator()<B, 5>();        \
    break;
  switch (bits) {
    DDG_GROUPED_CASE(3) DDG_GROUPED_CASE(4) DDG_GROUPED_CASE(5) DDG_GROUPED_CASE(6) DDG_GROUPED_CASE(7)
  }
#undef DDG_GROUPED_CASE
}


// Several M > 64 products: workgroup i runs tile i - tile_start[j] of product
// j with that product's bit width.
__global__ __launch_bounds__(512, 1) void gemm_grouped_large_kernel(GroupLargeArgs ga) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kLdsStage];
  const int bid = blockIdx.x;
  int j = 0;
  while (j + 1 < ga.count && bid >= ga.tile_start[j + 1]) ++j;
  j = __builtin_amdgcn_readfirstlane(j);
  const int t = bid - ga.tile_start[j];
  switch (ga.bits[j]) {
    case 3: large_tile<3>(ga.g[j], t, lds); break;
    case 4: large_tile<4>(ga.g[j], t, lds); break;
    case 5: large_tile<5>(ga.g[j], t, lds); break;
    case 6: large_tile<6>(ga.g[j], t, lds); break;
    case 7: large_tile<7>(ga.g[j], t, lds); break;
  }
}

// Several products with 16 < M <= 16 RB: workgroup i runs workgroup
// i - wg_start[j] of product j (32 output columns: two column waves, a
// two-way K split) with that product's bit width.
template <int RB>
__global__ __launch_bounds__(256) void gemm_grouped_small_kernel(GroupArgs ga) {
  __shared__ SmallLds<RB, 2, 2> L;
  const int bid = blockIdx.x;
  int j = 0;
  while (j + 1 < ga.count && bid >= ga.wg_start[j + 1]) ++j;
  j = __builtin_amdgcn_readfirstlane(j);
  const int wg = bid - ga.wg_start[j];
  switch (ga.bits[j]) {
    case 3: small_body<3, RB, 2, 2>(ga.g[j], wg, L); break;
    case 4: small_body<4, RB, 2, 2>(ga.g[j], wg, L); break;
    case 5: small_body<5, RB, 2, 2>(ga.g[j], wg, L); break;
    case 6: small_body<6, RB, 2, 2>(ga.g[j], wg, L); break;
    case 7: small_body<7, RB, 2, 2>(ga.g[j], wg, L); break;
  }
}

hipError_t launch_gemm_grouped_small(const GroupArgs& ga, int rb, hipStream_t stream) {
  if (ga.count < 1 || ga.count > kMaxGroup) return hipErrorInvalidValue;
  const int wgs = ga.wg_start[ga.count];
  if (wgs <= 0) return hipSuccess;
  if (rb == 2)
    gemm_grouped_small_kernel<2><<<dim3((unsigned)wgs), dim3(256), 0, stream>>>(ga);
  else if (rb == 4)
    gemm_grouped_small_kernel<4><<<dim3((unsigned)wgs), dim3(256), 0, stream>>>(ga);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm_grouped_large(const GroupLargeArgs& ga, hipStream_t stream) {
  if (ga.count < 1 || ga.count > kMaxGroup) return hipErrorInvalidValue;
  const int tiles = ga.tile_start[ga.count];
  if (tiles <= 0) return hipSuccess;
  gemm_grouped_large_kernel<<<dim3((unsigned)tiles), dim3(512), 0, stream>>>(ga);
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(const GroupArgs& ga, hipStream_t stream) {
  if (ga.count < 1 || ga.count > kMaxGroup) return hipErrorInvalidValue;
  const int wgs = ga.wg_start[ga.count];
  if (wgs <= 0) return hipSuccess;
  if (ga.ncb == 4)
    gemm_grouped_skinny_kernel<4><<<dim3((unsigned)wgs), dim3(512), 0, stream>>>(ga);
  else if (ga.ncb == 2)
    gemm_grouped_skinny_kernel<2><<<dim3((unsigned)wgs), dim3(512), 0, stream>>>(ga);
  else if (ga.ncb == 1)
    gemm_grouped_skinny_kernel<1><<<dim3((unsigned)wgs), dim3(512), 0, stream>>>(ga);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ddg
