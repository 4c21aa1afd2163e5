// FP4 weights x FP8 activations (W4A8) on the gfx950 scaled matrix
// instructions (the FP4DiT article: 4-bit floating-point weight formats in
// groups of 128, §3.2.1 / §4.1; 8-bit per-token activations, §3.2.3):
//   fp4_quantize_pack_kernel  per-group(128) scale + nearest 4-bit level, packed
//                             two codes per byte (even index in the low nibble)
//   fp8_quantize_rows_kernel  per-token scale + E4M3 round-to-nearest-even
//   w4a8_gemm_kernel          Y = s_x[m] sum_g s_w[n,g] (X_q W_q^T)_g
#include "ddg_launch.hpp"

namespace ddg {

namespace {

// Magnitudes by index, and the midpoints between neighbours (exact in float32).
//   E2M1: 0 .5 1 1.5 2 3 4 6    E3M0: 0 .25 .5 1 2 4 8 16    E1M2: 0 .25 .. 1.75
template <int FMT>
struct Fp4Fmt;
template <>
struct Fp4Fmt<kFp4E2M1> {
  static constexpr float vmax = 6.0f;
  static constexpr float mid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
};
template <>
struct Fp4Fmt<kFp4E3M0> {
  static constexpr float vmax = 16.0f;
  static constexpr float mid[7] = {0.125f, 0.375f, 0.75f, 1.5f, 3.0f, 6.0f, 12.0f};
};
template <>
struct Fp4Fmt<kFp4E1M2> {
  static constexpr float vmax = 1.75f;
  static constexpr float mid[7] = {0.125f, 0.375f, 0.625f, 0.875f, 1.125f, 1.375f, 1.625f};
};

// E4M3 bytes of the 8 magnitudes of each 4-bit format (all exact in E4M3),
// as two little-endian words: magnitudes 0-3, 4-7.
template <int FMT>
struct Fp4AsE4M3;
template <>
struct Fp4AsE4M3<kFp4E2M1> {   // 0 .5 1 1.5 | 2 3 4 6
  static constexpr uint32_t lo = 0x3C383000u, hi = 0x4C484440u;
};
template <>
struct Fp4AsE4M3<kFp4E3M0> {   // 0 .25 .5 1 | 2 4 8 16
  static constexpr uint32_t lo = 0x38302800u, hi = 0x58504840u;
};
template <>
struct Fp4AsE4M3<kFp4E1M2> {   // 0 .25 .5 .75 | 1 1.25 1.5 1.75
  static constexpr uint32_t lo = 0x34302800u, hi = 0x3E3C3A38u;
};

// Eight 4-bit codes (code i in bits 4i) -> eight E4M3 bytes in code order.
template <int FMT>
__device__ __forceinline__ u32x2 fp4_codes_to_e4m3(uint32_t x) {
  const uint32_t ev = x & 0x0F0F0F0Fu;                 // codes 0 2 4 6, one per byte
  const uint32_t od = (x >> 4) & 0x0F0F0F0Fu;          // codes 1 3 5 7
  auto conv = [](uint32_t c) {
    const uint32_t mag = __builtin_amdgcn_perm(Fp4AsE4M3<FMT>::hi, Fp4AsE4M3<FMT>::lo, c & 0x07070707u);
    return mag | ((c & 0x08080808u) << 4);
  };
  const uint32_t e = conv(ev), o = conv(od);
  u32x2 r;
  r[0] = __builtin_amdgcn_perm(o, e, 0x05010400u);    // e0 o0 e1 o1
  r[1] = __builtin_amdgcn_perm(o, e, 0x07030602u);    // e2 o2 e3 o3
  return r;
}

// Index of the level nearest a (>= 0): count the midpoints below it; on a
// midpoint move up only to an even index.
template <int FMT>
__device__ __forceinline__ uint32_t fp4_index(float a) {
  uint32_t idx = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const float mj = Fp4Fmt<FMT>::mid[j];
    idx += (a > mj || (a == mj && ((j + 1) & 1) == 0)) ? 1u : 0u;
  }
  return idx;
}

// One lane per 32 consecutive weights; the four lanes of a 128-group share
// the abs-max through a quad butterfly.  Output: 4 dwords of codes per lane
// (code 8 j + i in bits 4 i of dword j) and one scale per group.
template <int FMT, bool F32_IN>
__global__ __launch_bounds__(256) void fp4_quantize_pack_kernel(const void* __restrict__ w,
                                                               int64_t n_chunks,
                                                               uint32_t* __restrict__ packed,
                                                               float* __restrict__ scales) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = c < n_chunks;
  const int64_t cc = valid ? c : n_chunks - 1;               // whole quads past the end
  float v[32];
  if constexpr (F32_IN) {
    const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(w) + cc * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 t = src[i];
      v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
    }
  } else {
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(w) + cc * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 t = src[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bf16_bits_to_f32(t[j] & 0xFFFFu);
        v[8 * i + 2 * j + 1] = bf16_bits_to_f32(t[j] >> 16);
      }
    }
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
  a = __builtin_fmaxf(a, __shfl_xor(a, 1));
  a = __builtin_fmaxf(a, __shfl_xor(a, 2));
  const float s = a / Fp4Fmt<FMT>::vmax;
  const bool zero = !(s != 0.0f);
  u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float r = zero ? 0.0f : v[i] / s;
    const uint32_t idx = fp4_index<FMT>(__builtin_fabsf(r));
    const uint32_t code = idx | ((r < 0.0f && idx != 0u) ? 8u : 0u);
    out[i >> 3] |= code << (4 * (i & 7));
  }
  if (valid) {
    reinterpret_cast<u32x4*>(packed)[c] = out;
    if ((threadIdx.x & 3) == 0) scales[c >> 2] = zero ? 0.0f : s;
  }
}

// E4M3 code of a finite float: clamp to +-448, round to nearest even
// (subnormals: multiples of 2^-9; normals: three mantissa bits).
__device__ __forceinline__ uint32_t e4m3_code(float r) {
  const float a = __builtin_fminf(__builtin_fabsf(r), 448.0f);
  uint32_t mag;
  if (a < 0.015625f) {
    mag = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    uint32_t b = __builtin_bit_cast(uint32_t, a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    mag = ((((b >> 23) - 127u + 7u) & 15u) << 3) | ((b >> 20) & 7u);
  }
  return (mag != 0u && r < 0.0f) ? (mag | 0x80u) : mag;
}

// One wave per row (four rows per workgroup): the row's abs-max, then
// r = x / s and its E4M3 code, eight codes per lane and step.
__global__ __launch_bounds__(256) void fp8_quantize_rows_kernel(const uint16_t* __restrict__ x,
                                                               int64_t m, int k,
                                                               uint8_t* __restrict__ q,
                                                               float* __restrict__ sx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + row * k);
  const int chunks = k / 8;
  float a = 0.0f;
  for (int c = lane; c < chunks; c += 64) {
    const u32x4 t = src[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a = __builtin_fmaxf(a, __builtin_fabsf(bf16_bits_to_f32(t[j] & 0xFFFFu)));
      a = __builtin_fmaxf(a, __builtin_fabsf(bf16_bits_to_f32(t[j] >> 16)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off));
  const float s = a / 448.0f;
  const bool zero = !(s != 0.0f);
  u32x2* dst = reinterpret_cast<u32x2*>(q + row * k);
  for (int c = lane; c < chunks; c += 64) {
    const u32x4 t = src[c];
    u32x2 o = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t h = (j & 1) ? (t[j >> 1] >> 16) : (t[j >> 1] & 0xFFFFu);
      const float r = zero ? 0.0f : bf16_bits_to_f32(h) / s;
      o[j >> 2] |= e4m3_code(r) << (8 * (j & 3));
    }
    dst[c] = o;
  }
  if (lane == 0) sx[row] = zero ? 0.0f : s;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16e __attribute__((ext_vector_type(16)));

// X tile per 128-group: 256 rows x 128 bytes of E4M3 (32 KB); row r holds
// its 16-byte chunk c at slot c ^ (r & 7), so that the eight lanes of a
// ds_read_b128 phase (eight consecutive rows, one chunk) hit distinct banks.
constexpr int kW8Stage = 256 * 128;

// Workgroup = 8 waves, tile 256 rows x 256 columns; wave w owns columns
// 32w .. 32w + 31 for all 256 rows (8 row blocks of 32).  Per 128-group and
// row block: two v_mfma_scale_f32_32x32x64_f8f6f4 (A = X as E4M3 from LDS,
// B = the packed codes from the weight rows, unit block scales)
// accumulate the group's partial sum, which is then scaled by the column's
// group scale into the running fp32 accumulator.  A: lane half h holds the
// bytes of k 32 h .. 32 h + 31 of a 64-wide step; B: see load_w below.
template <int FMT>
__global__ __launch_bounds__(512, 1) void w4a8_gemm_kernel(W4A8Args args) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kW8Stage];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lh = lane >> 5;
  int tm, tn;
  tile_coords(blockIdx.x, args.tiles_m, args.tiles_n, tm, tn);
  const int m0 = tm * 256;
  const int nw0 = tn * 256;
  const int K = args.k;
  const int G = K / 128;
  const uint32_t wrow = (uint32_t)K / 2;
  const int m_valid = min(256, args.m - m0);
  const int n_valid = min(256, args.n - nw0);
  const rsrc_t rx = make_rsrc(args.xq + (int64_t)m0 * K, (uint32_t)m_valid * (uint32_t)K);
  const rsrc_t rw = make_rsrc(args.packed + (int64_t)nw0 * wrow, (uint32_t)n_valid * wrow);
  const rsrc_t rs = make_rsrc(args.wscales + (int64_t)nw0 * G, (uint32_t)n_valid * G * 4);

  // X -> LDS: DMA i (0..3) of wave w fills 1 KB block 4w + i: rows
  // 8 (4w + i) + lane/8, slot lane%8 holding chunk slot ^ (row & 7).
  uint32_t xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * (4 * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    xoff[i] = (uint32_t)r * (uint32_t)K + (uint32_t)c * 16;
  }
  auto issue_x = [&](int g, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (lds_ptr_t)(lds + stage * kW8Stage + (4 * wave + i) * 1024), 16, xoff[i],
          (uint32_t)g * 128, 0, 0);
  };
  // The lane's column and its 32 codes per 64-wide step.
  //  * E2M1 runs as an FP4 B operand: lane half h carries k 16h .. 16h + 15 of
  //    the step in its first 16 nibbles and k 32 + 16h .. 32 + 16h + 15 in the
  //    other 16 (the pairing with A's k 32h' + e was read off the instruction
  //    with one-hot operands): two 8-byte pieces of the packed row, at byte
  //    offsets 8h and 16 + 8h.
  //  * E3M0 and E1M2 are not matrix formats; their values are exact in E4M3,
  //    so B is FP8, which pairs like A: lane half h takes the 16 bytes (codes
  //    32h .. 32h + 31) at offset 16h, converted through a byte lookup.
  constexpr bool kNative = FMT == kFp4E2M1;
  const uint32_t ncol = (uint32_t)(32 * wave + lr);
  const uint32_t woff = ncol * wrow + (kNative ? 8u : 16u) * (uint32_t)lh;
  const uint32_t soff = ncol * (uint32_t)G * 4;
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  auto load_w = [&](int g, u32x4 (&b)[2], float& sc) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if constexpr (kNative) {
        const v2u lo = __builtin_amdgcn_raw_buffer_load_b64(rw, woff + 32u * ks, (uint32_t)g * 64, 0);
        const v2u hi = __builtin_amdgcn_raw_buffer_load_b64(rw, woff + 32u * ks + 16u, (uint32_t)g * 64, 0);
        b[ks][0] = lo.x; b[ks][1] = lo.y; b[ks][2] = hi.x; b[ks][3] = hi.y;
      } else {
        b[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff + 32u * ks,
                                                                                (uint32_t)g * 64, 0));
      }
    }
    sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff, (uint32_t)g * 4, 0));
  };
  auto read_a = [&](int stage, int rb, int ks) __attribute__((always_inline)) -> i32x8 {
    const int r = rb * 32 + lr;
    const int c0 = 4 * ks + 2 * lh;
    const uint8_t* base = lds + stage * kW8Stage + r * 128;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + ((c0 ^ (r & 7)) * 16));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + (((c0 + 1) ^ (r & 7)) * 16));
    i32x8 a;
    a[0] = (int)lo[0]; a[1] = (int)lo[1]; a[2] = (int)lo[2]; a[3] = (int)lo[3];
    a[4] = (int)hi[0]; a[5] = (int)hi[1]; a[6] = (int)hi[2]; a[7] = (int)hi[3];
    return a;
  };

  f32x16e acc[8];
#pragma unroll
  for (int rb = 0; rb < 8; ++rb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[rb][i] = 0.0f;
  f32x16e zero16;
#pragma unroll
  for (int i = 0; i < 16; ++i) zero16[i] = 0.0f;

  u32x4 bc[2], bn[2];
  float sc = 0.0f, sn = 0.0f;
  issue_x(0, 0);
  load_w(0, bc, sc);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int stage = 0;
  // the last group fetches itself again into the idle stage (never read), so
  // that the loop body stays one straight block
  for (int g = 0; g < G; ++g) {
    const int gn = min(g + 1, G - 1);
    issue_x(gn, stage ^ 1);
    load_w(gn, bn, sn);
    i32x8 b0, b1;
    if constexpr (kNative) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b0[j] = (int)bc[0][j]; b0[j + 4] = 0;
        b1[j] = (int)bc[1][j]; b1[j + 4] = 0;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 c0 = fp4_codes_to_e4m3<FMT>(bc[0][j]);
        const u32x2 c1 = fp4_codes_to_e4m3<FMT>(bc[1][j]);
        b0[2 * j] = (int)c0[0]; b0[2 * j + 1] = (int)c0[1];
        b1[2 * j] = (int)c1[0]; b1[2 * j + 1] = (int)c1[1];
      }
    }
    constexpr int kBFmt = kNative ? 4 : 0;                // B as FP4 (E2M1) or FP8 (E4M3)
    // row block rb: its A reads were issued one block earlier; its partial sum
    // is scaled into acc while the next block's MFMAs run
    i32x8 a0 = read_a(stage, 0, 0), a1 = read_a(stage, 0, 1);
    f32x16e tp;
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
      i32x8 n0, n1;
      if (rb < 7) {
        n0 = read_a(stage, rb + 1, 0);
        n1 = read_a(stage, rb + 1, 1);
      }
      f32x16e t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, zero16, 0, kBFmt, 0, 127, 0, 127);
      t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, t, 0, kBFmt, 0, 127, 0, 127);
      if (rb > 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[rb - 1][i] = __builtin_fmaf(tp[i], sc, acc[rb - 1][i]);
      }
      tp = t;
      if (rb < 7) {
        a0 = n0;
        a1 = n1;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[7][i] = __builtin_fmaf(tp[i], sc, acc[7][i]);
    __builtin_amdgcn_s_waitcnt(0);             // the next group's X and weights have landed
    __syncthreads();                           // ... and every wave is done with this stage
    bc[0] = bn[0];
    bc[1] = bn[1];
    sc = sn;
    stage ^= 1;
  }

  // Epilogue: lane holds rows 8(r/4) + 4h + r%4 of column lane%32, r = 0..15.
  const int col = nw0 + 32 * wave + lr;
  if (col < args.n) {
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + rb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row < args.m) {
          const float v = acc[rb][r] * args.xscales[row];
          if (args.out_bf16)
            static_cast<__bf16*>(args.y)[(int64_t)row * args.n + col] = (__bf16)v;
          else
            static_cast<float*>(args.y)[(int64_t)row * args.n + col] = v;
        }
      }
    }
  }
}

template <int FMT>
hipError_t launch_fp4_quant(const void* w, bool f32_in, int64_t n_chunks, uint32_t* packed,
                            float* scales, hipStream_t stream) {
  const dim3 grid((unsigned)((n_chunks + 255) / 256)), block(256);
  if (f32_in)
    fp4_quantize_pack_kernel<FMT, true><<<grid, block, 0, stream>>>(w, n_chunks, packed, scales);
  else
    fp4_quantize_pack_kernel<FMT, false><<<grid, block, 0, stream>>>(w, n_chunks, packed, scales);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp4_quantize_pack(const void* w, bool f32_in, int64_t n_chunks, int fmt,
                                    uint32_t* packed, float* scales, hipStream_t stream) {
  switch (fmt) {
    case kFp4E2M1: return launch_fp4_quant<kFp4E2M1>(w, f32_in, n_chunks, packed, scales, stream);
    case kFp4E3M0: return launch_fp4_quant<kFp4E3M0>(w, f32_in, n_chunks, packed, scales, stream);
    case kFp4E1M2: return launch_fp4_quant<kFp4E1M2>(w, f32_in, n_chunks, packed, scales, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fp8_quantize_rows(const uint16_t* x, int64_t m, int k, uint8_t* q, float* sx,
                                    hipStream_t stream) {
  if (m == 0) return hipSuccess;
  fp8_quantize_rows_kernel<<<dim3((unsigned)((m + 3) / 4)), dim3(256), 0, stream>>>(x, m, k, q, sx);
  return hipGetLastError();
}

hipError_t launch_w4a8_gemm(const W4A8Args& a, int fmt, hipStream_t stream) {
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(512);
  switch (fmt) {
    case kFp4E2M1: w4a8_gemm_kernel<kFp4E2M1><<<grid, block, 0, stream>>>(a); return hipGetLastError();
    case kFp4E3M0: w4a8_gemm_kernel<kFp4E3M0><<<grid, block, 0, stream>>>(a); return hipGetLastError();
    case kFp4E1M2: w4a8_gemm_kernel<kFp4E1M2><<<grid, block, 0, stream>>>(a); return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace ddg
