// Launcher of the low-rank pre-pass T = bf16(X L1) (bit-width independent).
#include "ddg_launch.hpp"

namespace ddg {

hipError_t launch_lowrank_t(const __bf16* x, const __bf16* lora_down, __bf16* t, int m, int k,
                            int r, hipStream_t stream) {
  const dim3 grid((unsigned)((m + 15) / 16)), block(64 * kLowrankWaves);
  switch ((r + 15) / 16) {
    case 1: lowrank_t_kernel<1><<<grid, block, 0, stream>>>(x, lora_down, t, m, k, r); break;
    case 2: lowrank_t_kernel<2><<<grid, block, 0, stream>>>(x, lora_down, t, m, k, r); break;
    case 3: lowrank_t_kernel<3><<<grid, block, 0, stream>>>(x, lora_down, t, m, k, r); break;
    case 4: lowrank_t_kernel<4><<<grid, block, 0, stream>>>(x, lora_down, t, m, k, r); break;
    case 5: lowrank_t_kernel<5><<<grid, block, 0, stream>>>(x, lora_down, t, m, k, r); break;
    case 6: lowrank_t_kernel<6><<<grid, block, 0, stream>>>(x, lora_down, t, m, k, r); break;
    case 7: lowrank_t_kernel<7><<<grid, block, 0, stream>>>(x, lora_down, t, m, k, r); break;
    case 8: lowrank_t_kernel<8><<<grid, block, 0, stream>>>(x, lora_down, t, m, k, r); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ddg
