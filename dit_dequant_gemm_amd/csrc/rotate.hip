// Random-permuted block-Hadamard rotation of rows (the OrbitQuant article,
// §2.1 rotation, §2.2 offline weights / online activations):
//   out[r, b h + j] = sum_t H_h[j, t] / sqrt(h) * sign[b h + t] * x[r, perm[b h + t]]
// with H_h the Sylvester Walsh-Hadamard matrix.  HBM-bound: one read and one
// write of every row; the permutation table stays in LDS.
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "ddg_launch.hpp"

namespace ddg {

namespace {

// Table entry (32 bits): byte offset of the source element in a row buffer
// (entries outside [0, d) point at a zero slot just past the row), and the
// sign in bit 31.
constexpr uint32_t kNegBit = 0x80000000u;
constexpr uint32_t kOffMask = 0x7FFFFFFFu;

// Row buffer: the row, rounded up to whole 1 KB DMA instructions, plus 16
// bytes; the zero slot sits right after the row.
__host__ __device__ constexpr uint32_t rot_buf_bytes(uint32_t row_bytes) {
  return ((row_bytes + 1023u) & ~1023u) + 16u;
}

// s_waitcnt vmcnt(v), no wait on the other counters; v (0..63) need not be a
// compile-time constant (one immediate per value).
__device__ __forceinline__ void wait_vmcnt(int v) {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (void)((v == I ? (__builtin_amdgcn_s_waitcnt(0x0F70 | (I & 15) | ((I >> 4) << 14)), true)
                   : false) || ...);
  }(std::make_integer_sequence<int, 64>{});
}

// Value of the lane whose index differs from this lane's in bit M (M = 1, 2,
// ..., 32).  Strides within a row of 16 lanes use DPP moves (quad_perm for 1
// and 2; a half-row or row mirror followed by a quad_perm for 4 and 8), 16 a
// ds_swizzle bit pattern, 32 a ds_bpermute.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  const int x = __builtin_bit_cast(int, v);
  int y;
  if constexpr (M == 1) {
    y = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);          // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    y = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);          // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    const int t = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);  // i ^ 7 (half-row mirror)
    y = __builtin_amdgcn_mov_dpp(t, 0x1B, 0xF, 0xF, false);             // ^ 3 (quad_perm [3,2,1,0])
  } else if constexpr (M == 8) {
    const int t = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);  // i ^ 15 (row mirror)
    y = __builtin_amdgcn_mov_dpp(t, 0x141, 0xF, 0xF, false);            // ^ 7 (half-row mirror)
  } else if constexpr (M == 16) {
    y = __builtin_amdgcn_ds_swizzle(x, 0x401F);                      // and 0x1F, xor 0x10
  } else {
    y = __builtin_amdgcn_ds_bpermute((int)((threadIdx.x & 63) ^ 32) << 2, x);
  }
  return __builtin_bit_cast(float, y);
}

// A workgroup of W (2..8) waves takes steps of rps consecutive rows: step k of
// workgroup g covers rows (g + k gridDim.x) rps + i, i < rps.  Wave 0 is the
// producer: it only moves rows HBM -> LDS with buffer_load ... lds, so its
// waits count its own loads alone.  Waves 1..W-1 are consumers: they gather,
// transform and store, and never wait for memory, so their stores stream out.
// A ring of nb (1..4) steps' row buffers lets the producer keep up to nb - 1
// steps in flight while the consumers work on the oldest; one barrier per step
// hands a step over (with one, a second barrier returns it).  A job is 1024
// consecutive outputs of one row, lane l holding the 16 outputs c0 + 16 l + t:
// butterfly strides 1..8 run in registers, strides 16 .. h/2 across lanes
// (lane xor 1 .. h/32); consumer c takes jobs c, c + W - 1, ... of the step.
template <bool F32_IN, bool F32_OUT, int LH>
__global__ __launch_bounds__(512) void rpbh_rotate_kernel(const void* __restrict__ x, int64_t n,
                                                         int d, const int32_t* __restrict__ perm,
                                                         const int8_t* __restrict__ signs,
                                                         float rs, int nb, int rps,
                                                         void* __restrict__ out) {
  using RowT = typename std::conditional<F32_IN, float, uint16_t>::type;
  constexpr int H = 1 << LH;
  constexpr int kEs = sizeof(RowT);
  extern __shared__ __attribute__((aligned(1024))) uint8_t rot_lds[];
  uint32_t* tab = reinterpret_cast<uint32_t*>(rot_lds);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int consumers = (int)(blockDim.x >> 6) - 1;
  const uint32_t data_bytes = (uint32_t)d * kEs;
  const uint32_t buf_bytes = rot_buf_bytes(data_bytes);
  uint8_t* bufs = rot_lds + (size_t)d * 4;
  const int slots = nb * rps;

  for (int i = tid; i < d; i += blockDim.x) {
    const int p = perm[i];
    uint32_t e = (uint32_t)((p >= 0 && p < d) ? p : d) * kEs;
    if (signs[i] < 0) e |= kNegBit;
    tab[i] = e;
  }
  if (tid < 4 * slots)
    reinterpret_cast<uint32_t*>(bufs + (tid >> 2) * buf_bytes + data_bytes)[tid & 3] = 0u;
  lds_barrier();

  const int dmas = (int)((data_bytes + 1023u) >> 10);        // 1 KB per instruction
  const int64_t steps = (n + rps - 1) / rps;
  auto rows_in = [&](int64_t step) -> int {                   // rows of a step that exist
    return (int)std::min<int64_t>(rps, n - step * rps);
  };
  auto load_step = [&](int64_t step, int b) __attribute__((always_inline)) {
    const int rows = rows_in(step);
    for (int i = 0; i < rows; ++i) {
      const rsrc_t rx = make_rsrc(static_cast<const RowT*>(x) + (step * rps + i) * d, data_bytes);
      uint8_t* dst = bufs + (b * rps + i) * buf_bytes;
      for (int j = 0; j < dmas; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(dst + j * 1024), 16,
                                                 (uint32_t)(j * 1024 + lane * 16), 0, 0, 0);
    }
  };

  const int64_t stride = gridDim.x;
  if (wave == 0) {
    for (int j = 0; j < (nb > 1 ? nb - 1 : 1); ++j)
      if ((int64_t)blockIdx.x + j * stride < steps) load_step(blockIdx.x + j * stride, j);
  }
  const int jobs_per_row = (d + 1023) >> 10;
  int b = 0;
  for (int64_t k = blockIdx.x; k < steps; k += stride) {
    if (wave == 0) {
      // this step has landed; the loads of the (at most nb - 2) steps after it may not have
      int pend = 0;
      for (int j = 1; j <= nb - 2; ++j)
        if (k + j * stride < steps) pend += rows_in(k + j * stride) * dmas;
      wait_vmcnt(pend < 64 ? pend : 0);
    }
    lds_barrier();                                         // ... for every wave; the oldest step's buffers are free
    if (wave == 0) {
      const int64_t next = k + (int64_t)(nb - 1) * stride;
      if (nb > 1 && next < steps) load_step(next, (b + nb - 1) % nb);
    } else {
      const int jobs = rows_in(k) * jobs_per_row;
      for (int job = wave - 1; job < jobs; job += consumers) {
        const int ri = job / jobs_per_row;
        const int c0 = (job - ri * jobs_per_row) * 1024;
        const uint8_t* row = bufs + (b * rps + ri) * buf_bytes;
        const int64_t r = k * rps + ri;
        const int e0 = c0 + 16 * lane;                     // this lane's first output
        const bool valid = e0 < d;                         // a short last job leaves lanes idle
        float v[16];
        if (valid) {
          const u32x4* tp = reinterpret_cast<const u32x4*>(tab + e0);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const u32x4 t = tp[q4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t off = t[q] & kOffMask, sg = t[q] & kNegBit;
              uint32_t bits;
              if constexpr (F32_IN)
                bits = *reinterpret_cast<const uint32_t*>(row + off);
              else
                bits = (uint32_t)*reinterpret_cast<const uint16_t*>(row + off) << 16;
              v[4 * q4 + q] = __builtin_bit_cast(float, bits ^ sg);
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 16; ++q) v[q] = 0.0f;
        }
        // strides 1, 2, 4, 8 (below h) in registers
#pragma unroll
        for (int st = 1; st < 16 && st < H; st <<= 1) {
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            if ((q & st) == 0) {
              const float a = v[q], bb = v[q + st];
              v[q] = a + bb;
              v[q + st] = a - bb;
            }
          }
        }
        // strides 16 .. h/2 across lanes: the lower lane of a pair takes the
        // sum, the upper one the difference (partner - own)
        auto cross = [&]<int M>(std::integral_constant<int, M>) __attribute__((always_inline)) {
          if constexpr (16 * M < H) {
            const float sgn = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = __builtin_fmaf(sgn, v[q], lane_xor<M>(v[q]));
          }
        };
        cross(std::integral_constant<int, 1>{});
        cross(std::integral_constant<int, 2>{});
        cross(std::integral_constant<int, 4>{});
        cross(std::integral_constant<int, 8>{});
        cross(std::integral_constant<int, 16>{});
        cross(std::integral_constant<int, 32>{});
        if (valid) {
          const int64_t o = r * d + e0;
          if constexpr (F32_OUT) {
            f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(out) + o);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              f32x4 w;
              w[0] = v[4 * q] * rs; w[1] = v[4 * q + 1] * rs; w[2] = v[4 * q + 2] * rs; w[3] = v[4 * q + 3] * rs;
              dst[q] = w;
            }
          } else {
            u32x4* dst = reinterpret_cast<u32x4*>(static_cast<__bf16*>(out) + o);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              u32x4 w;
#pragma unroll
              for (int p2 = 0; p2 < 4; ++p2)
                w[p2] = pack_bf16x2(v[8 * q + 2 * p2] * rs, v[8 * q + 2 * p2 + 1] * rs);
              dst[q] = w;
            }
          }
        }
      }
    }
    if (nb > 1) {
      b = b + 1 == nb ? 0 : b + 1;
    } else {
      lds_barrier();                                       // the consumers are done with the buffers
      if (wave == 0 && k + stride < steps) load_step(k + stride, 0);
    }
  }
}

template <bool FI, bool FO, int LH>
hipError_t launch_h(const void* x, int64_t n, int d, const int32_t* perm, const int8_t* signs,
                    float rs, void* out, int cus, hipStream_t stream) {
  auto kern = rpbh_rotate_kernel<FI, FO, LH>;
  // allow the whole LDS once per device (one bit per device)
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(raised.load(std::memory_order_acquire) & bit)) {
    if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit))
      return e;
    raised.fetch_or(bit, std::memory_order_acq_rel);
  }
  const size_t tab = (size_t)d * 4;
  const size_t one = rot_buf_bytes((uint32_t)d * (FI ? 4 : 2));
  if (tab + one > (size_t)kLdsLimit) return hipErrorInvalidValue;
  // eight waves (seven consumers); rows per step: enough 1024-output jobs for
  // the consumers (<= 7 rows); ring depth two where it fits, else one;
  // workgroups per CU: as many as the LDS holds (<= 4), never more than steps.
  // (A sweep of 4/8 waves, 1/2 rows per step and rings of 2..4 at 4096 x 3072
  // spans 16.9 .. 22.6 us; this is its fastest corner.)
  const int jobs_per_row = (d + 1023) / 1024;
  int rps = (int)std::max<int64_t>(1, std::min<int64_t>(7 / jobs_per_row, n));
  while (rps > 1 && tab + 2 * rps * one > (size_t)kLdsLimit) --rps;
  const int nb = (int)std::min<size_t>(2, (kLdsLimit - tab) / (rps * one));
  const size_t lds = tab + (size_t)nb * rps * one;
  const int per_cu = (int)std::min<size_t>(4, kLdsLimit / lds);
  const int64_t steps = (n + rps - 1) / rps;
  const int64_t grid = std::min<int64_t>(steps, (int64_t)cus * per_cu);
  kern<<<dim3((unsigned)grid), dim3(512), lds, stream>>>(x, n, d, perm, signs, rs, nb, rps, out);
  return hipGetLastError();
}

template <bool FI, bool FO>
hipError_t launch_io(const void* x, int64_t n, int d, const int32_t* perm, const int8_t* signs, int h,
                     float rs, void* out, int cus, hipStream_t stream) {
  switch (h) {
    case 2: return launch_h<FI, FO, 1>(x, n, d, perm, signs, rs, out, cus, stream);
    case 4: return launch_h<FI, FO, 2>(x, n, d, perm, signs, rs, out, cus, stream);
    case 8: return launch_h<FI, FO, 3>(x, n, d, perm, signs, rs, out, cus, stream);
    case 16: return launch_h<FI, FO, 4>(x, n, d, perm, signs, rs, out, cus, stream);
    case 32: return launch_h<FI, FO, 5>(x, n, d, perm, signs, rs, out, cus, stream);
    case 64: return launch_h<FI, FO, 6>(x, n, d, perm, signs, rs, out, cus, stream);
    case 128: return launch_h<FI, FO, 7>(x, n, d, perm, signs, rs, out, cus, stream);
    case 256: return launch_h<FI, FO, 8>(x, n, d, perm, signs, rs, out, cus, stream);
    case 512: return launch_h<FI, FO, 9>(x, n, d, perm, signs, rs, out, cus, stream);
    case 1024: return launch_h<FI, FO, 10>(x, n, d, perm, signs, rs, out, cus, stream);
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
