// Random-permuted block-Hadamard rotation of rows (the OrbitQuant article,
// §2.1 rotation, §2.2 offline weights / online activations):
//   out[r, b h + j] = sum_t H_h[j, t] / sqrt(h) * sign[b h + t] * x[r, perm[b h + t]]
// with H_h the Sylvester Walsh-Hadamard matrix.  HBM-bound: one read and one
// write of every row; the permutation table stays in LDS.
#include <algorithm>
#include <atomic>

#include "ddg_launch.hpp"

namespace ddg {

namespace {

constexpr uint32_t kNegBit = 0x80000000u;   // table entry: negative sign
constexpr uint32_t kZeroBit = 0x40000000u;  // table entry: index outside [0, d), reads as 0

// One workgroup (4 waves) takes rows blockIdx.x, blockIdx.x + gridDim.x, ...
// LDS: the table (d words: permuted index and sign) and one row as float32.
// A wave job covers E * 64 consecutive outputs (E = h / 64 for h >= 64, else 1:
// then 64 / h whole blocks): lane l holds outputs c0 + 64 j + l, j < E, so the
// butterfly strides below 64 run across lanes and the others in registers.
template <bool F32_IN, bool F32_OUT, int E>
__global__ __launch_bounds__(256) void rpbh_rotate_kernel(const void* __restrict__ x, int64_t n,
                                                         int d, const int32_t* __restrict__ perm,
                                                         const int8_t* __restrict__ signs, int h,
                                                         float rs, void* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint32_t rot_lds[];
  uint32_t* tab = rot_lds;
  float* row = reinterpret_cast<float*>(rot_lds + d);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int C = 64 * E;

  for (int i = tid; i < d; i += 256) {
    const int p = perm[i];
    uint32_t e = (p >= 0 && p < d) ? (uint32_t)p : kZeroBit;
    if (signs[i] < 0) e |= kNegBit;
    tab[i] = e;
  }

  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    __syncthreads();                       // the table is ready; the last row is consumed
    if constexpr (F32_IN) {
      const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + r * d);
      for (int i = tid; i < d / 4; i += 256) reinterpret_cast<f32x4*>(row)[i] = src[i];
    } else {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + r * d);
      for (int i = tid; i < d / 8; i += 256) {
        const u32x4 v = src[i];
        f32x4 lo, hi;
        lo[0] = bf16_bits_to_f32(v[0] & 0xFFFFu); lo[1] = bf16_bits_to_f32(v[0] >> 16);
        lo[2] = bf16_bits_to_f32(v[1] & 0xFFFFu); lo[3] = bf16_bits_to_f32(v[1] >> 16);
        hi[0] = bf16_bits_to_f32(v[2] & 0xFFFFu); hi[1] = bf16_bits_to_f32(v[2] >> 16);
        hi[2] = bf16_bits_to_f32(v[3] & 0xFFFFu); hi[3] = bf16_bits_to_f32(v[3] >> 16);
        reinterpret_cast<f32x4*>(row)[2 * i] = lo;
        reinterpret_cast<f32x4*>(row)[2 * i + 1] = hi;
      }
    }
    __syncthreads();

    for (int c0 = wave * C; c0 < d; c0 += 4 * C) {
      float v[E];
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const uint32_t t = tab[c0 + 64 * j + lane];
        const float a = (t & kZeroBit) ? 0.0f : row[t & (kZeroBit - 1)];
        v[j] = (t & kNegBit) ? -a : a;
      }
      // strides 1 .. min(h, 64) / 2 across lanes: the lower index of a pair
      // takes the sum, the upper one the difference
      for (int s = 1; s < 64 && s < h; s <<= 1) {
        const bool upper = (lane & s) != 0;
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const float o = __shfl_xor(v[j], s);
          v[j] = upper ? o - v[j] : v[j] + o;
        }
      }
      // strides 64 .. h / 2 in registers
#pragma unroll
      for (int js = 1; js < E; js <<= 1) {
#pragma unroll
        for (int j = 0; j < E; ++j) {
          if ((j & js) == 0) {
            const float a = v[j], b = v[j + js];
            v[j] = a + b;
            v[j + js] = a - b;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int64_t o = r * d + c0 + 64 * j + lane;
        const float y = v[j] * rs;
        if constexpr (F32_OUT)
          static_cast<float*>(out)[o] = y;
        else
          static_cast<__bf16*>(out)[o] = (__bf16)y;
      }
    }
  }
}

template <bool FI, bool FO, int E>
hipError_t launch_e(const void* x, int64_t n, int d, const int32_t* perm, const int8_t* signs, int h,
                    float rs, void* out, int cus, hipStream_t stream) {
  const size_t lds = (size_t)d * 8;
  auto kern = rpbh_rotate_kernel<FI, FO, E>;
  // allow the largest table + row once per device (one bit per device)
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(raised.load(std::memory_order_acquire) & bit)) {
    if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           kRotateMaxD * 8))
      return e;
    raised.fetch_or(bit, std::memory_order_acq_rel);
  }
  // as many workgroups per CU as the LDS allows (at most 8), never more than rows
  const int per_cu = (int)std::min<size_t>(8, (size_t)kLdsLimit / lds);
  const int64_t grid = std::min<int64_t>(n, (int64_t)cus * std::max(per_cu, 1));
  kern<<<dim3((unsigned)grid), dim3(256), lds, stream>>>(x, n, d, perm, signs, h, rs, out);
  return hipGetLastError();
}

template <bool FI, bool FO>
hipError_t launch_io(const void* x, int64_t n, int d, const int32_t* perm, const int8_t* signs, int h,
                     float rs, void* out, int cus, hipStream_t stream) {
  switch (h <= 64 ? 1 : h / 64) {
    case 1: return launch_e<FI, FO, 1>(x, n, d, perm, signs, h, rs, out, cus, stream);
    case 2: return launch_e<FI, FO, 2>(x, n, d, perm, signs, h, rs, out, cus, stream);
    case 4: return launch_e<FI, FO, 4>(x, n, d, perm, signs, h, rs, out, cus, stream);
    case 8: return launch_e<FI, FO, 8>(x, n, d, perm, signs, h, rs, out, cus, stream);
    case 16: return launch_e<FI, FO, 16>(x, n, d, perm, signs, h, rs, out, cus, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rpbh_rotate(const void* x, bool f32_in, int64_t n, int d, const int32_t* perm,
                              const int8_t* signs, int h, void* out, bool f32_out, int cus,
                              hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const float rs = (float)(1.0 / __builtin_sqrt((double)h));
  if (f32_in)
    return f32_out ? launch_io<true, true>(x, n, d, perm, signs, h, rs, out, cus, stream)
                   : launch_io<true, false>(x, n, d, perm, signs, h, rs, out, cus, stream);
  return f32_out ? launch_io<false, true>(x, n, d, perm, signs, h, rs, out, cus, stream)
                 : launch_io<false, false>(x, n, d, perm, signs, h, rs, out, cus, stream);
}

}  // namespace ddg
