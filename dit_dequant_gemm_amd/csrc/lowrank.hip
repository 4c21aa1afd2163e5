// Launcher of the low-rank pre-pass T = bf16(X L1) (bit-width independent).
#include "ddg_launch.hpp"

namespace ddg {

namespace {
constexpr int kLowrankCUs = 256;      // compute units of the MI355X

template <int RBLK, int RR>
hipError_t launch_t(const __bf16* x, const __bf16* lora_down, __bf16* t, int m, int k, int r,
                    hipStream_t stream) {
  const dim3 grid((unsigned)((m + 16 * RR - 1) / (16 * RR))), block(64 * kLowrankWaves);
  lowrank_t_kernel<RBLK, RR><<<grid, block, 0, stream>>>(x, lora_down, t, m, k, r);
  return hipGetLastError();
}

template <int RBLK>
hipError_t launch_rblk(const __bf16* x, const __bf16* lora_down, __bf16* t, int m, int k, int r,
                       int rr, hipStream_t stream) {
  if constexpr (RBLK <= 2) {
    if (rr == 4) return launch_t<RBLK, 4>(x, lora_down, t, m, k, r, stream);
  }
  if constexpr (RBLK <= 4) {
    if (rr == 2) return launch_t<RBLK, 2>(x, lora_down, t, m, k, r, stream);
  }
  return launch_t<RBLK, 1>(x, lora_down, t, m, k, r, stream);
}
}  // namespace

// Row blocks of 16 per workgroup of the pre-pass for m rows at rank r.
int lowrank_t_row_blocks(int m, int r) {
  const int rblk = (r + 15) / 16;
  // several row blocks per workgroup while the grid keeps two workgroups per
  // compute unit (4096 x 3072, r = 32: one block 12.7 us, two 18.8, four
  // 23.7; 32760 x 5120: 145, 109, 86 us)
  for (int c = 4; c > 1; c /= 2)
    if (c * rblk <= 8 && (m + 16 * c - 1) / (16 * c) >= 2 * kLowrankCUs) return c;
  // (more waves per workgroup for grids that leave units idle were no faster:
  // 16 x 5120 at r = 32 took 15.1 us with 16 waves against 14.8 with 4)
  return 1;
}

hipError_t launch_lowrank_t(const __bf16* x, const __bf16* lora_down, __bf16* t, int m, int k,
                            int r, hipStream_t stream) {
  const int rr = lowrank_t_row_blocks(m, r);
  switch ((r + 15) / 16) {
    case 1: return launch_rblk<1>(x, lora_down, t, m, k, r, rr, stream);
    case 2: return launch_rblk<2>(x, lora_down, t, m, k, r, rr, stream);
    case 3: return launch_rblk<3>(x, lora_down, t, m, k, r, rr, stream);
    case 4: return launch_rblk<4>(x, lora_down, t, m, k, r, rr, stream);
    case 5: return launch_rblk<5>(x, lora_down, t, m, k, r, rr, stream);
    case 6: return launch_rblk<6>(x, lora_down, t, m, k, r, rr, stream);
    case 7: return launch_rblk<7>(x, lora_down, t, m, k, r, rr, stream);
    case 8: return launch_rblk<8>(x, lora_down, t, m, k, r, rr, stream);
    default: return hipErrorInvalidValue;
  }
}

int lowrank_split_chunks(int k, int* gpc) {
  const int g = k / kGroup;
  *gpc = (g + 31) / 32;
  return (g + *gpc - 1) / *gpc;
}

namespace {
template <int RBLK>
hipError_t launch_part(const __bf16* x, const __bf16* lora_down, float* part, int m, int k, int r,
                       int gpc, int chunks, hipStream_t stream) {
  const dim3 grid((unsigned)((m + 15) / 16), (unsigned)chunks), block(64 * kLowrankWaves);
  lowrank_t_part_kernel<RBLK><<<grid, block, 0, stream>>>(x, lora_down, part, m, k, r, gpc);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_lowrank_t_split(const __bf16* x, const __bf16* lora_down, __bf16* t, float* part,
                                  int m, int k, int r, hipStream_t stream) {
  int gpc = 1;
  const int chunks = lowrank_split_chunks(k, &gpc);
  hipError_t e = hipErrorInvalidValue;
  switch ((r + 15) / 16) {
    case 1: e = launch_part<1>(x, lora_down, part, m, k, r, gpc, chunks, stream); break;
    case 2: e = launch_part<2>(x, lora_down, part, m, k, r, gpc, chunks, stream); break;
    case 3: e = launch_part<3>(x, lora_down, part, m, k, r, gpc, chunks, stream); break;
    case 4: e = launch_part<4>(x, lora_down, part, m, k, r, gpc, chunks, stream); break;
    case 5: e = launch_part<5>(x, lora_down, part, m, k, r, gpc, chunks, stream); break;
    case 6: e = launch_part<6>(x, lora_down, part, m, k, r, gpc, chunks, stream); break;
    case 7: e = launch_part<7>(x, lora_down, part, m, k, r, gpc, chunks, stream); break;
    case 8: e = launch_part<8>(x, lora_down, part, m, k, r, gpc, chunks, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const int64_t n4 = (int64_t)m * r / 4;
  lowrank_t_reduce_kernel<0><<<dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream>>>(part, t, m, r, chunks);
  return hipGetLastError();
}

}  // namespace ddg
